// ra_kernels.h -- kernel argument blocks and host-side launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "ra_common.h"

namespace ra {

struct QKPrologueArgs {
  const void* q;      // [B, N, H, D] bf16 or f32
  const void* k;
  uint8_t* q_out;     // int4: [B*H, nblk] 64-token fp6 e2m3 tiles (48 D bytes each); bf16 path: [B*H, Npad, D] bf16
  uint8_t* k_out;
  float* s_q;         // [B*H, nblk] (int4 path only)
  float* s_k;
  RopeTabs tabs;
  int B, N, H, Npad, nblk;
};

struct VAmaxArgs {
  const void* v;
  uint32_t* vamax;    // [B*H, D] float bits of the per-channel max |v|
  int N, H, chunk;
};

struct VQuantArgs {
  const void* v;
  const uint32_t* vamax;
  uint8_t* v_out;     // int4: [B*H, nkb] 64-key fp6 e2m3 tiles (48 D bytes each); bf16: [B*H, nkb, D, 64] bf16
  float* s_v;         // [B*H, D]
  int N, H, nkb;
};

// The P map's thresholds as the attention kernels use them ([RA] Sec. 4.2:
// u = round(P p) with p = 2^d, P = 15 or 7).  With x = -d >= 0, u = #{k :
// x <= X_k}, X_k the largest binary32 value with P 2^-X_k >= k + 1/2.  The
// kernels sort x into cells j = rint(x * 4096) (ties to even) and keep one
// byte per cell in a table, stored in reverse at address top - j, with
// every j >= top (no code above 0 there) at address 0.  cell[k] is the
// cell holding X_k; bit k of `split` is set when that cell also holds
// values above X_k (the table then cannot decide, and the kernel compares
// y = x / 8 with ythr[k] = X_k / 8, both exact).
constexpr int kPTabEntries = 20112;   // table bytes: top + 1 <= this for P = 15 and 7
// The table as the kernels hold it in LDS (at address 0): kPTabBytes bytes
// of entries, then 16 records of 8 bytes.  The host builds it once per plan
// (pmap_table in ra_host.cpp) and uploads it with the RoPE tables; every
// workgroup copies it into LDS.  Entry of address a (cell j = top - a): u,
// the number of X_k whose cell lies above j plus the X_k whose cell is j
// when that cell holds nothing above X_k, as the e4m3 byte of u; a cell that
// holds X_k and values above it is marked 0x80 | k.  Record k < P: X_k / 8
// (binary32), then the e4m3 bytes of k and k + 1 and two zero bytes;
// records k >= P are zero.
constexpr int kPTabBytes = (kPTabEntries + 15) & ~15;
constexpr int kPThrBytes = 16 * 8;
constexpr int kPTabTotal = kPTabBytes + kPThrBytes;   // a multiple of 16
struct PMapArgs {
  int cell[15];
  float ythr[15];
  uint32_t split;
  int P;              // 15 (range-optimized) or 7 (symmetric)
  int top;            // even, above cell[0]
  float top_sub;      // top * 2^-149 (a binary32 subnormal)
};

struct AttnArgs {
  const uint8_t* qp;  // Q / K / V code bytes (int4) or bf16 tensors (bf16 path)
  const uint8_t* kp;
  const uint8_t* vp;
  const float* s_q;
  const float* s_k;
  const float* s_v;
  void* out;          // [B, N, H, D] f32 or bf16
  int N, H, Npad, nblk, nkb, nqt;
  float alpha;        // f32(log2(e) * softmax_scale): log2 units per unit of scaled score
  int p_mode;         // 0: range-optimized P (u = round(15 p), code u - 8); 1: symmetric (u = code = round(7 p))
  int v_hadamard;     // V codes are of V H (H = Walsh-Hadamard / sqrt D): the output is multiplied by H
  PMapArgs pm;        // int4 path
  const uint8_t* ptab; // int4 path: the P-map table (kPTabTotal bytes, 16-byte aligned)
  uint32_t* row_dbg;  // row fingerprints of the parity variant of the int4 kernel ([B*H*N][4]), else null
};

struct TileDumpArgs {
  int32_t* s_int;     // [64, 64]
  int8_t* p_code;     // [64, 64]
  int32_t* pv_int;    // [64, D]
  float* m_after;     // [64]
  int bh, q_blk, kv_blk;
};

void launch_int4_prologue(const QKPrologueArgs& qa, const VAmaxArgs& va, const VQuantArgs& vq,
                          int D, int rot, bool in_bf16, bool v_hadamard, hipStream_t st);
void launch_bf16_prologue(const QKPrologueArgs& qa, const VQuantArgs& vq, int D, bool in_bf16,
                          hipStream_t st);
void launch_int4_attn(const AttnArgs& a, int D, bool out_bf16, int B, hipStream_t st);
void launch_int4_tile_dump(const AttnArgs& a, const TileDumpArgs& t, int D, hipStream_t st);
void launch_int4_attn_rowdbg(const AttnArgs& a, int D, int B, hipStream_t st);
void launch_pmap_probe(const float* d, uint8_t* u, int64_t n, const PMapArgs& pm, const uint8_t* ptab,
                       hipStream_t st);
void launch_bf16_attn(const AttnArgs& a, int D, bool out_bf16, int B, hipStream_t st);
void launch_copy(void* dst, const void* src, size_t bytes, hipStream_t st);

// Device address of the current device's no-allocation workspace
// (ra_noalloc.hip).
hipError_t noalloc_scratch(void** ptr);

// Operand types of the matrix-core throughput kernel (ra_peak.hip).
enum PeakKind { kPeakI8 = 0, kPeakFp8 = 1, kPeakFp6 = 2, kPeakFp6Fp8 = 3, kPeakBf16 = 4 };
void launch_mfma_peak(int kind, int iters, int blocks, float* sink, uint64_t* clk, hipStream_t st);
int mfma_peak_ops_per_instr(int kind);   // 0 for an unknown kind
int mfma_peak_chains();                  // independent MFMAs per wave per iteration

}  // namespace ra
