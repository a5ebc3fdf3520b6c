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

struct AttnArgs {
  const uint8_t* qp;  // Q / K / V code bytes (int4) or bf16 tensors (bf16 path)
  const uint8_t* kp;
  const uint8_t* vp;
  const float* s_q;
  const float* s_k;
  const float* s_v;
  void* out;          // [B, N, H, D] f32 or bf16
  int N, H, Npad, nblk, nkb, nqt;
  float alpha_g;      // f32(log2(e) * softmax_scale * kPGrid)   (int4 path)
  float alpha;        // f32(log2(e) * softmax_scale)            (bf16 path)
  int p_mode;         // 0: range-optimized P (u = round(15 p), code u - 8); 1: symmetric (u = code = round(7 p))
  int v_hadamard;     // V codes are of V H (H = Walsh-Hadamard / sqrt D): the output is multiplied by H
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
void launch_pmap_probe(const float* x, uint8_t* u, int64_t n, int p_mode, hipStream_t st);
void launch_bf16_attn(const AttnArgs& a, int D, bool out_bf16, int B, hipStream_t st);
void launch_copy(void* dst, const void* src, size_t bytes, hipStream_t st);

// Operand types of the matrix-core throughput kernel (ra_peak.hip).
enum PeakKind { kPeakI8 = 0, kPeakFp8 = 1, kPeakFp6 = 2, kPeakFp6Fp8 = 3, kPeakBf16 = 4 };
void launch_mfma_peak(int kind, int iters, int blocks, float* sink, uint64_t* clk, hipStream_t st);
int mfma_peak_ops_per_instr(int kind);   // 0 for an unknown kind
int mfma_peak_chains();                  // independent MFMAs per wave per iteration

}  // namespace ra
