// ra_int4_attn.hip -- INT4 FlashAttention forward with range-optimized P.
//
// Method source: "RotateAttention: RoPE-Aware Rotation and Range Rectification
// for INT4 Quantized Attention in Video Generation" (pith.science review):
// abstract (INT4 Q, K, V inside FlashAttention; P = exp(QK - max QK)) and
// Sec. 4.2 (P mapped onto the full signed INT4 range: code = round(15 p) - 8;
// the symmetric quantization it replaces, code = round(7 p) in [0, 7], as the
// ablation mode p_mode = 1).
//
// gfx950 design
//   * One workgroup = 12 waves = 384 query rows of one (b, h); each wave owns
//     32 queries.  A wave fits in 168 VGPRs, so three waves share each SIMD
//     and hide one another's LDS and matrix-core latencies (one workgroup per
//     CU).  Workgroup ids are remapped so that the workgroups resident on one
//     XCD walk the same head, sharing K/V tiles in that XCD's L2.
//   * Per 64-key step the K and V code tiles (6 KB of fp6 each for D = 128)
//     are copied from global memory straight into LDS by buffer loads with
//     the LDS-direct bit (16 bytes per lane, no VGPRs, no VALU), as they lie.
//     Ten stages of each; the workgroup barrier is taken once every five
//     steps.
//   * S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 with both operands fp6 e2m3
//     (exact for |code| <= 7, and twice the fp8 rate); every partial sum is
//     an integer below 2^24, so the fp32 accumulator holds the exact integer
//     score and no int->float conversion is needed.  Each lane holds one
//     query column, so the row max is in-lane (+1 cross-half swap).
//   * P codes come straight out of the accumulator registers: the exponent
//     d = f32(S c - m) of each score (one FMA) is turned into a table index
//     j = rint(-4096 d) by a multiply into the fp32 subnormal range (whose
//     bit pattern is then the rounded index), and looked up in a 20 KB byte
//     table of u = round(15 2^d) as e4m3 at LDS address 0 (stored in
//     reverse, built once per plan on the host and copied into LDS by each
//     workgroup).  Fifteen table
//     cells hold a rounding boundary of 15 2^d inside them; their entries
//     are marked, and the few scores that land in one are decided exactly by
//     an fp32 compare of d against the boundary.  Two byte permutes and an
//     OR pack four codes in the order the PV MFMA wants them as its B
//     operand; V is stored pre-permuted to match.
//   * PV = V^T P^T runs on the same MFMA with V in fp6 and P in fp8 (u in
//     [0, 15] is exact in e4m3, and a step's sums are integers below 2^24),
//     so each step's PV is exact; it accumulates across steps in fp32
//     registers, scaled by beta only when a query's running max rises (rare
//     after the first few steps).  The row sum of the codes is one more MFMA
//     per step (16x16x128, the same P operand against an fp4 0/1 selector),
//     so it costs no VALU work and lands in every lane that owns the query.
#include <type_traits>

#include "ra_common.h"
#include "ra_kernels.h"

namespace ra {

constexpr int kWaves = 12;                 // waves per workgroup
constexpr int kQTile = 32 * kWaves;        // query rows per workgroup
constexpr int kSync = 5;                   // steps per workgroup barrier
constexpr int kStages = 2 * kSync;         // LDS stages of K and of V tiles
constexpr int kSkLds = 5120;               // key steps whose K scales are held in LDS (N <= 327,680)

template <int D>
struct Cfg {
  static constexpr int QC = D / 64;        // 64-channel chunks of the Q.K contraction
  static constexpr int DT = D / 32;        // 32-channel tiles of O
  static constexpr int KT = qk6_tile_bytes(D);   // fp6 K tile of 64 keys (48 D bytes)
  static constexpr int VT = v6_tile_bytes(D);   // fp6 V tile of 64 keys (48 D bytes)
};

template <int D>
struct State {
  v16f acc[Cfg<D>::DT];     // O^T: sum of u * vhat, scaled by beta when m rises
  float m;                  // running max (log2 units), this lane's query
  v4f lsum;                 // row sum of u (16x16 MFMA accumulator; every register = this query's)
};

// ---- range-optimized P map through an LDS table --------------------------
//
// For a score S with scale c and running max m (log2 units), the exponent
// is d = f32(S c - m) and u = round(P 2^d) = #{k : x <= X_k} with x = -d
// (PMapArgs).  With c' = c / 8 and m' = m / 8 (exact power-of-two scalings):
//   y = clamp(fma(S, -c', m'))   f32(m - S c) / 8 = x / 8, clamped to
//                                [0, 1]: keys at or above the running max
//                                (d >= 0) give 0, the top code; with the
//                                DX10 clamp mode of compute kernels a NaN
//                                or a -0 becomes +0
//   w = clamp(fma(y, -2^-134, top 2^-149))
//                                a subnormal (f32 denormals are enabled in
//                                these kernels) of spacing 2^-149: the sum
//                                rounds top - 4096 x to the nearest
//                                integer, ties to even, and the clamp sends
//                                every negative result to +0, so
//                                bits(w) = max(top - rint(4096 x), 0)
// The table sits at LDS address 0 and bits(w) is the byte address of the
// entry of cell j = rint(4096 x), stored in reverse: address top - j, and
// address 0 for every j >= top, where u = 0.  All keys that far below the
// running max (most keys of a long row) read the same byte, a broadcast.
// Scalings by 1/8 are exact unless a value is below 2^-123, and then x is
// far below the smallest X_k and every path gives u = P.  The running max
// is passed as m' + 0, which turns a -0 into +0.
//
// The entry of cell j is e4m3(u) when every x of the cell has the same u;
// in the cell of an X_k that also holds values above it, the entry is
// 0x80 | k (no e4m3 code of 0..15 has bit 7 set) and u = k + (y <= X_k / 8),
// decided by pmap_fix after the lookup from the 8-byte record k behind the
// table: X_k / 8, then the bytes e4m3(k) and e4m3(k + 1).
constexpr float kPIdxScale = 0.125f;                        // 2^-3
constexpr uint32_t kPSplit = 0x80808080u;                   // marked entries, per packed byte

__device__ __forceinline__ float pmap_y(float s, float c2, float m2) {
  // med3(x, 0, 1) folds into the clamp bit of the FMA (DX10 clamp mode).
  return __builtin_amdgcn_fmed3f(__builtin_fmaf(s, -c2, m2), 0.0f, 1.0f);
}

__device__ __forceinline__ uint32_t ptab_addr(float s, float c2, float m2, float top_sub) {
  return __float_as_uint(__builtin_amdgcn_fmed3f(__builtin_fmaf(pmap_y(s, c2, m2), -0x1p-134f, top_sub), 0.0f, 1.0f));
}

// e4m3 encoding of an integer 0 <= u <= 15 (exact).
__device__ __forceinline__ uint32_t e4m3_of_uint(uint32_t u) {
  if (u == 0u) return 0u;
  const uint32_t e = 31u - (uint32_t)__builtin_clz(u);       // floor(log2 u) <= 3
  return ((e + 7u) << 3) | ((u << (3u - e)) & 7u);
}

// Inverse of e4m3_of_uint (debug dumps).
__device__ __forceinline__ uint32_t e4m3_to_uint(uint32_t b) {
  if (b == 0u) return 0u;
  const uint32_t e = (b >> 3) - 7u, m = b & 7u;
  return ((8u | m) << e) >> 3;
}

// ---- K/V staging: global memory -> LDS without registers ------------------

typedef __attribute__((address_space(3))) uint8_t lds_u8;
// 16-byte buffer load with the LDS-direct bit: lane i copies 16 bytes from
// base(rsrc) + voffset into LDS at lds + 16 i (lds is wave-uniform).  It is
// written as an instruction the compiler does not model as a store to LDS:
// the modelled form makes the compiler wait for every copy in flight before
// any LDS read it cannot prove disjoint from the copy's target, which here
// is every read of the other stages.  Completion is ordered explicitly by
// wait_lds_dma() and the workgroup barrier; no register receives data, and
// M0 is set and used inside the statement.
__device__ __forceinline__ void lds_copy16(v4i rsrc, uint32_t lds, int voffset) {
  const uint32_t m = lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m), "v"(voffset), "s"(rsrc)
               : "memory");
}

// Buffer descriptor over `bytes` bytes at `base` (reads past the end return 0).
__device__ __forceinline__ v4i make_rsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
             __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)), (int)bytes, 0x00020000};
}

__device__ __forceinline__ void wait_lds_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The P-map table (entries and records, kPTabTotal bytes, built by the host)
// into the LDS array `tab` by the NW waves of the workgroup: 16 bytes per
// lane, 64 lanes per instruction, lanes past the end masked off.  Complete
// after wait_lds_dma() and a barrier.  The copies' LDS address is formed
// from the array's own address, so the compiler knows the copy statement
// may write it (an LDS array it saw no store to could otherwise be read as
// undefined).
template <int NW>
__device__ __forceinline__ void ptab_copy(const uint8_t* g, uint8_t* tab) {
  constexpr int kChunks = kPTabTotal / 16;
  static_assert(kPTabTotal % 16 == 0, "whole 16-byte chunks");
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)tab;
  const v4i rsrc = make_rsrc(g, kPTabTotal);
  for (int c = wave; 64 * c < kChunks; c += NW)
    if (64 * c + lane < kChunks) lds_copy16(rsrc, base + (uint32_t)(1024 * c), 1024 * c + 16 * lane);
}

// Copies of one step's K tile and V tile (fp6, 48 D bytes each) by NW
// waves.  The tiles are cut into 16-byte slots numbered in LDS order; a wave
// copies 64 consecutive slots per instruction, K slots first.  Both tiles
// are copied as they lie.
template <int D, int NW>
struct TileDma {
  static constexpr int KS = Cfg<D>::KT / 16;
  static constexpr int VS = Cfg<D>::VT / 16;
  static constexpr int NI = (KS + VS + 64 * NW - 1) / (64 * NW);
  static_assert(KS % 64 == 0 && VS % 64 == 0, "tiles must be whole waves of slots");

  // Per instruction j (all step-invariant): this lane's source byte offset
  // within its tile, and, uniform over the wave, which tile the wave's 64
  // slots belong to (0 none, 1 K, 2 V) and their byte offset in the stage.
  int off[NI];
  int kind[NI];
  int lds[NI];

  __device__ __forceinline__ TileDma() {
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int first = (j * NW + wave) * 64;
      if (first >= KS + VS) {
        kind[j] = 0;
        lds[j] = 0;
        off[j] = 0;
      } else if (first < KS) {
        kind[j] = 1;
        lds[j] = first * 16;
        off[j] = (first + lane) * 16;
      } else {
        kind[j] = 2;
        lds[j] = (first - KS) * 16;
        off[j] = (first - KS + lane) * 16;
      }
      kind[j] = __builtin_amdgcn_readfirstlane(kind[j]);
      lds[j] = __builtin_amdgcn_readfirstlane(lds[j]);
    }
  }

  // K tile at kt -> kst, V tile at vt -> vst (global addresses of the
  // tiles); a null tile is skipped.
  __device__ __forceinline__ void issue(const uint8_t* kt, const uint8_t* vt, uint32_t kst, uint32_t vst) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      if (kind[j] == 1 && kt != nullptr)
        lds_copy16(make_rsrc(kt, Cfg<D>::KT), kst + lds[j], off[j]);
      else if (kind[j] == 2 && vt != nullptr)
        lds_copy16(make_rsrc(vt, Cfg<D>::VT), vst + lds[j], off[j]);
    }
  }
};

// Q operands (B operand of S^T = K Q^T on the f8f6f4 MFMA, fp6): query `q`,
// channels 64qc + 32hf + 0..31, i.e. channel group 2qc + hf of its tile.
template <int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int bh, int q, int hf,
                                       v8i (&qop)[Cfg<D>::QC]) {
#pragma unroll
  for (int qc = 0; qc < Cfg<D>::QC; ++qc) {
    v4i lo = v4i{0, 0, 0, 0};
    v2i hi = v2i{0, 0};
    if (q < a.Npad) {
      const uint8_t* t = a.qp + ((size_t)bh * a.nblk + (q >> 6)) * Cfg<D>::KT;
      lo = *reinterpret_cast<const v4i*>(t + qk6_lo_off(q & 63, 2 * qc + hf));
      hi = *reinterpret_cast<const v2i*>(t + qk6_hi_off(D, q & 63, 2 * qc + hf));
    }
    qop[qc] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
  }
}

// Key index (within the 64-key step) of accumulator register r of M-tile mt.
__device__ __forceinline__ int acc_key(int mt, int r, int hf) {
  return mt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
}

// LDS address of a lane's base for one step's reads, hidden from the
// optimizer: otherwise it splits stage + lane + constant offsets into one
// loop-invariant register per read and re-adds the stage offset to each,
// instead of one add per base and the constants in the read instructions.
typedef __attribute__((address_space(3))) const uint8_t lds_cu8;
__device__ __forceinline__ lds_cu8* lds_base(uint32_t a) { return (lds_cu8*)a; }
// A stage's LDS address as an opaque scalar: the compiler can neither fold
// it into the per-lane offsets (one loop-invariant register per unrolled
// step and operand) nor hoist the one add per operand and step.
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}
template <typename T>
__device__ __forceinline__ T lds_ld(lds_cu8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
// Compiler-only fence after the reads of one fp6 operand: otherwise the
// 8-byte reads of two operands are merged into one ds_read2_b64, whose
// result then has to be moved next to each operand's 16-byte part (the six
// registers of an fp6 operand must be consecutive).  No instruction.
__device__ __forceinline__ void operand_fence() { asm volatile("" ::: "memory"); }

// ---- building blocks of one 64-key step for the 32 queries of a wave ------

// S^T of the step (exact integers in fp32): kst is the step's fp6 K tile.
// Lane (ln, hf) supplies key row 32mt + ln, channel group 2qc + hf: one
// 16-byte and one 8-byte LDS read, consecutive rows at consecutive
// addresses (no bank conflicts without a swizzle).  Both offsets are linear
// in (row, group), so one lane base per part plus constants covers all reads.
template <int D>
__device__ __forceinline__ void qk_step(uint32_t kst, const v8i (&qop)[Cfg<D>::QC], v16f (&s)[2]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  lds_cu8* const klo = lds_base(kst + qk6_lo_off(ln, hf));
  lds_cu8* const khi = lds_base(kst + qk6_hi_off(D, ln, hf));
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mt][r] = 0.0f;
#pragma unroll
    for (int qc = 0; qc < Cfg<D>::QC; ++qc) {
      const int rg = 128 * qc + 32 * mt;   // (64 g + row) - (64 hf + ln)
      const v4i lo = lds_ld<v4i>(klo + 16 * rg);
      const v2i hi = lds_ld<v2i>(khi + 8 * rg);
      operand_fence();
      const v8i ka = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
      s[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qop[qc], s[mt], 2, 2, 0, 0, 0, 0);
    }
  }
}

// Keys at or past `nvalid` (ragged last step) get S = -inf: they drop out of
// the max and map to u = 0.  The mask runs only on the ragged last key step;
// its argument is passed through opaque_sgpr() so that the compiler can
// neither hoist the 32 key comparisons out of that branch nor if-convert the
// masking into selects executed on every step.
__device__ __forceinline__ int opaque_sgpr(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

__device__ __forceinline__ void mask_scores(v16f (&s)[2], int nvalid) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (acc_key(mt, r, hf) >= nvalid) s[mt][r] = -INFINITY;
}

// New running max for this lane's query (log2 units): the larger of m and
// f32(max_j S_j * c) (rounded to nearest; + 0 makes a -0 product +0, so
// that the max never has to order zeros of both signs).
__device__ __forceinline__ float running_max(const v16f (&s)[2], float c, float m) {
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int k = 2; k < 32; ++k) mx = fmaxf(mx, s[k >> 4][k & 15]);
  return fmaxf(m, xhalf_max_f(mx) * c + 0.0f);
}

// P codes of a whole step (u in e4m3, both M-tiles) in the order of the PV
// MFMA's B operand: register 4i+e of M-tile mt goes to byte e of p[mt][i].
// All 32 table loads are issued before any is used, so the LDS latency is
// paid once per step; each load leaves one byte in the low end of its
// register, and two v_perm (bytes 0-1 and 2-3) and an OR pack four of them.
// Marked entries (bit 7) still need pmap_fix.
__device__ __forceinline__ void pmap_step(const v16f (&s)[2], float c2, float m2, float top_sub,
                                          const uint8_t* tab, uint32_t (&p)[2][4]) {
  uint32_t x[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) x[k] = tab[ptab_addr(s[k >> 4][k & 15], c2, m2, top_sub)];
#pragma unroll
  for (int w = 0; w < 8; ++w)
    p[w >> 2][w & 3] = __builtin_amdgcn_perm(x[4 * w + 1], x[4 * w], 0x0C0C0400u) |
                       __builtin_amdgcn_perm(x[4 * w + 3], x[4 * w + 2], 0x04000C0Cu);
}

// Whether any lane of the wave holds a marked entry (wave-uniform).
__device__ __forceinline__ bool pmap_marked(const uint32_t (&p)[2][4]) {
  const uint32_t o = (p[0][0] | p[0][1] | p[0][2] | p[0][3]) | (p[1][0] | p[1][1] | p[1][2] | p[1][3]);
  return __builtin_amdgcn_ballot_w64((o & kPSplit) != 0u) != 0u;
}

// Decide the marked entries exactly: the entry 0x80 | k stands for
// u = k + (x <= X_k), i.e. k + (y <= X_k / 8) with y as in the lookup.  A
// packed word is revisited only when some lane has a marked byte in it; its
// four bytes are then decided without branches (unmarked bytes keep theirs).
__device__ __forceinline__ void pmap_fix(const v16f (&s)[2], float c2, float m2, const uint8_t* recs,
                                         uint32_t (&p)[2][4]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t pw = p[w >> 2][w & 3];
    if (__builtin_amdgcn_ballot_w64((pw & kPSplit) != 0u) != 0u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b = (pw >> (8 * e)) & 0xFFu;
        if (b & 0x80u) {
          const float thr = *reinterpret_cast<const float*>(recs + 8 * (b & 0x0Fu));
          const float y = pmap_y(s[w >> 2][4 * (w & 3) + e], c2, m2);
          const uint32_t nb = e4m3_of_uint((b & 0x0Fu) + (y <= thr ? 1u : 0u));
          pw = __builtin_amdgcn_perm(nb, pw, (0x03020100u & ~(0xFFu << (8 * e))) | (0x04u << (8 * e)));
        }
      }
      p[w >> 2][w & 3] = pw;
    }
  }
}

// The whole P map of a step: lookups, then the exact decision of marked
// entries when the wave has any (rare: 15 cells of 2^15).
__device__ __forceinline__ void pmap_codes(const v16f (&s)[2], float c2, float m2, float top_sub,
                                           const uint8_t* tab, uint32_t (&p)[2][4]) {
  pmap_step(s, c2, m2, top_sub, tab, p);
  if (__builtin_expect(pmap_marked(p), 0)) pmap_fix(s, c2, m2, tab + kPTabBytes, p);
}

// Zero the P codes of keys at or past nvalid (ragged last step).
__device__ __forceinline__ void mask_p(uint32_t (&p)[2][4], int nvalid) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = min(max(nvalid - (32 * mt + 8 * g + 4 * hf), 0), 4);
      p[mt][g] &= n >= 4 ? 0xFFFFFFFFu : ((1u << (8 * n)) - 1u);
    }
}

// Row sums of the step's P codes on one 16x16x128 MFMA.  B = the PV operand:
// lane l supplies column l % 16 with the 32 codes of query l % 32, so column
// n holds query n in lane groups 0 and 2 and query n + 16 in groups 1 and 3.
// A = fp4 0/1 selector.  An fp4 A lane covers, in registers 0-1, 16 K slots
// of an even B lane group and, in registers 2-3, 16 slots of an odd one
// (group 0: B groups 0 and 1, first 16 bytes; group 1: B groups 2 and 3,
// first 16; groups 2 and 3: the same with the last 16 bytes), so rows r with
// (r / 4) % 2 = 0 take ones in registers 0-1 and the others in registers
// 2-3.  Output row r of column n then sums all 64 keys of query
// n + 16 ((r / 4) % 2), the query of every lane that holds row r.
__device__ __forceinline__ v8i lsum_selector() {
  const int odd = (threadIdx.x >> 2) & 1;   // ((lane % 16) / 4) % 2
  const int one = 0x22222222;                 // fp4 e2m1 1.0 = 0x2
  return odd ? v8i{0, 0, one, one, 0, 0, 0, 0} : v8i{one, one, 0, 0, 0, 0, 0, 0};
}
// The selector rebuilt at its use (two selects), so that it occupies no
// registers between steps: the main loop has none to spare.
__device__ __forceinline__ v8i lsum_selector_at_use() {
  int odd = (threadIdx.x >> 2) & 1;
  asm volatile("" : "+v"(odd));
  const int one = 0x22222222;
  const int a = odd ? 0 : one, b = odd ? one : 0;
  return v8i{a, a, b, b, 0, 0, 0, 0};
}
__device__ __forceinline__ void lsum_step(const v8i& sel, const uint32_t (&p)[2][4], v4f& lsum) {
  const v8i pb = v8i{(int)p[0][0], (int)p[0][1], (int)p[0][2], (int)p[0][3],
                     (int)p[1][0], (int)p[1][1], (int)p[1][2], (int)p[1][3]};
  lsum = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pb, lsum, 4, 0, 0, 0, 0, 0);
}

// O^T += V^T P^T over the 64 keys of the step on the f8f6f4 MFMA with an
// fp6 A operand (V, cbsz 2) and an fp8 B operand (P).  Lane (ln, hf)
// supplies the fp6 string of channel 32 dt + ln, half hf: one 16-byte and
// one 8-byte read, tile dt 512 and 256 bytes past the lane bases.
template <int D>
__device__ __forceinline__ void pv_step(uint32_t vst, const uint32_t (&p)[2][4],
                                        v16f (&acc)[Cfg<D>::DT]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  const v8i pb = v8i{(int)p[0][0], (int)p[0][1], (int)p[0][2], (int)p[0][3],
                     (int)p[1][0], (int)p[1][1], (int)p[1][2], (int)p[1][3]};
  lds_cu8* const vlo = lds_base(vst + v6_lo_off(D, ln, hf));
  lds_cu8* const vhi = lds_base(vst + v6_hi_off(D, ln, hf));
  // All V operands are read before the first MFMA, so that the LDS latency
  // is paid once per step rather than once per MFMA.
  v8i va[Cfg<D>::DT];
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::DT; ++dt) {
    const v4i lo = lds_ld<v4i>(vlo + 512 * dt);
    const v2i hi = lds_ld<v2i>(vhi + 256 * dt);
    operand_fence();
    va[dt] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
  }
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::DT; ++dt)
    acc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[dt], pb, acc[dt], 2, 0, 0, 0, 0, 0);
}

// The running max rises from st.m to m_new: A = A * beta, L = (L + U) * beta.
// beta = 0 on the first step (st.m = -inf).
template <int D>
__device__ __forceinline__ void rescale(State<D>& st, float m_new) {
  const float beta = exp2f(st.m - m_new);
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[dt][r] *= beta;
  st.lsum *= beta;
}

// c = f32(f32(s_q s_k) alpha): log2 units per unit of integer score.
__device__ __forceinline__ float score_scale(float cq, float sk, float alpha) {
  const float sqk = cq * sk;
  return sqk * alpha;
}

// One whole 64-key step in program order (used by the parity dump kernel;
// the main kernel runs the same blocks software-pipelined).
template <int D, bool DUMP>
__device__ __forceinline__ void tile_step(uint32_t kst, uint32_t vst, const uint8_t* tab,
                                          const v8i (&qop)[Cfg<D>::QC], float cq, float alpha,
                                          float sk, int nvalid, State<D>& st,
                                          const TileDumpArgs* dump, int wave, int P, float top_sub) {
  const int zp = P == 15 ? 8 : 0;                  // code = u - zp
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  v16f s[2];
  qk_step<D>(kst, qop, s);
  if (nvalid < kBlock) mask_scores(s, nvalid);
  const float cp = score_scale(cq, sk, alpha);
  const float m_new = running_max(s, cp, st.m);
  if (__ballot(m_new > st.m) != 0) rescale<D>(st, m_new);
  st.m = m_new;
  uint32_t p[2][4];
  pmap_codes(s, cp * kPIdxScale, m_new * kPIdxScale + 0.0f, top_sub, tab, p);
  if (nvalid < kBlock) mask_p(p, nvalid);
  pv_step<D>(vst, p, st.acc);
  lsum_step(lsum_selector(), p, st.lsum);

  if (DUMP) {
    // Exact per-step integers: S, P codes (decoded from the e4m3 operand
    // bytes), PV = sum (u - zp) vhat = sum u vhat - zp sum vhat, running max.
    const int qrow = wave * 32 + ln;
    v16f pv[C::DT], cs[C::DT];
    uint32_t ones[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = acc_key(mt, r, hf);
        if (r % 4 == 0) ones[mt][r >> 2] = 0u;
        if (key < nvalid) ones[mt][r >> 2] |= 0x38u << (8 * (r & 3));   // e4m3 1.0
        const int sv = key < nvalid ? (int)s[mt][r] : 0;
        const int code = key < nvalid ? (int)e4m3_to_uint((p[mt][r >> 2] >> (8 * (r & 3))) & 0xFFu) - zp : -zp;
        dump->s_int[qrow * 64 + key] = sv;
        dump->p_code[qrow * 64 + key] = (int8_t)code;
      }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) { pv[dt][r] = 0.0f; cs[dt][r] = 0.0f; }
    pv_step<D>(vst, p, pv);
    pv_step<D>(vst, ones, cs);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = dt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        dump->pv_int[qrow * D + d] = (int)pv[dt][r] - zp * (int)cs[dt][r];
      }
    if (hf == 0) dump->m_after[qrow] = st.m;
  }
}

// Output side of the V-side Hadamard: o <- o H, H = Walsh-Hadamard / sqrt(D),
// over the 2 D/2 values of a query held by lanes l and l ^ 32 in O^T
// accumulator order (channel dt*32 + 8g + 4hf + e in register 4g + e of
// tile dt).  Butterflies over channel bits 0-1 (e), 2 (hf, across the two
// lanes), 3-4 (g) and 5.. (dt), then x 1/sqrt(D).  Part of the float path.
template <int D>
__device__ __forceinline__ void fwht_out(v16f (&acc)[Cfg<D>::DT]) {
  constexpr int DT = Cfg<D>::DT;
  auto bfly_r = [&](int bit) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!(r & bit)) {
          const float lo = acc[dt][r], hi = acc[dt][r + bit];
          acc[dt][r] = lo + hi;
          acc[dt][r + bit] = lo - hi;
        }
  };
  bfly_r(1);
  bfly_r(2);
  const bool upper = (threadIdx.x & 32) != 0;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float other = __shfl_xor(acc[dt][r], 32, 64);
      acc[dt][r] = upper ? other - acc[dt][r] : acc[dt][r] + other;
    }
  bfly_r(4);
  bfly_r(8);
#pragma unroll
  for (int bit = 1; bit < DT; bit <<= 1)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      if (!(dt & bit))
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float lo = acc[dt][r], hi = acc[dt + bit][r];
          acc[dt][r] = lo + hi;
          acc[dt + bit][r] = lo - hi;
        }
  const float sc = D == 128 ? 0.088388347648318440550f : 0.125f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] *= sc;
}

template <int D>
__device__ __forceinline__ void state_init(State<D>& st) {
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[dt][r] = 0.0f;
  st.m = -INFINITY;
  st.lsum = v4f{0.0f, 0.0f, 0.0f, 0.0f};
}

// Parity variant only: fingerprints of every P code of this lane's query
// (u = code + zero-point): the sum of u and the sum of u h(j) mod 2^32 with
// h(j) = 2654435761 (j + 1), j the key index.  Keys past N carry u = 0.
__device__ __forceinline__ void row_digest(const uint32_t (&p)[2][4], int t, uint32_t& ds, uint32_t& dh) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t u = e4m3_to_uint((p[mt][r >> 2] >> (8 * (r & 3))) & 0xFFu);
      const uint32_t key = (uint32_t)(t * kBlock + acc_key(mt, r, hf));
      ds += u;
      dh += u * (2654435761u * (key + 1u));
    }
}

__device__ __forceinline__ uint32_t xhalf_sum_u(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap((int)x, (int)x, false, false);
  return (uint32_t)r[0] + (uint32_t)r[1];
}

// DUMP: the parity variant -- the same kernel (same ring, barriers, peeled
// steps and workgroup order) that also writes, per query row, its final
// running max, the two P-code fingerprints and its row sum to a.row_dbg.
template <int D, bool OUT_BF16, bool VH, bool DUMP, bool SKL>
__global__ __launch_bounds__(64 * kWaves, 1) void k_int4_attn(AttnArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kPTabBytes + kPThrBytes + kStages * (C::KT + C::VT) +
                                                       (SKL ? 4 * kSkLds : 0)];
  uint8_t* const ptab = smem;                               // P-map table at LDS address 0
  float* const skl = reinterpret_cast<float*>(smem + kPTabBytes + kPThrBytes + kStages * (C::KT + C::VT));

  ptab_copy<kWaves>(a.ptab, ptab);                          // visible after the first barrier

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of (head, query-tile) ids.
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int full = nwg & ~7;
  const int lid = wg < full ? (wg & 7) * (full >> 3) + (wg >> 3) : wg;
  const int nqt = (a.N + kQTile - 1) / kQTile;
  const int bh = lid / nqt, qt = lid % nqt;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  const int q0 = qt * kQTile + wave * 32;
  const int qblk = q0 >> 6;
  const int nkb = a.nkb;

  v8i qop[C::QC];
  load_q<D>(a, bh, q0 + ln, hf, qop);
  const float cq = qblk < a.nblk ? a.s_q[(size_t)bh * a.nblk + qblk] : 0.0f;
  // K scales of this (b, h), one per key step.  SKL (at most kSkLds steps):
  // copied into LDS (visible after the first barrier) and each step reads
  // its successor's from there.  Otherwise each step loads it from global
  // memory (constant address space, a vector load), and waiting for that
  // load also waits for the tile copies the step has issued (about 1% slower
  // at 75,600 tokens).
  const __attribute__((address_space(4))) float* sk =
      (const __attribute__((address_space(4))) float*)(a.s_k + (size_t)bh * a.nblk);
  if constexpr (SKL)
    for (int i = threadIdx.x; i < nkb; i += 64 * kWaves) skl[i] = sk[i];

  State<D> st;
  state_init<D>(st);
  uint32_t dsum = 0, dhash = 0;                             // DUMP only

  // Step t: P x V of step t - 1 (its MFMAs are issued first and run while
  // the codes of step t are made from S in registers), the rescale the
  // accumulators need before P x V of step t, then S and the running max of
  // step t+1.  The other two waves on the SIMD fill the latencies.  K/V
  // tiles live in kStages = 2 kSync LDS stages and the workgroup barrier is
  // taken once every kSync steps (after the steps t with t % kSync == 0), so
  // the waves of a SIMD drift apart within a block of steps instead of
  // meeting in the same phase every step.  At step t each wave issues its
  // share of the copies of K of step t + kSync + 1 (read by step t + kSync
  // for S of step t + kSync + 1) and V of step t + kSync - 1 (read by step
  // t + kSync for P x V of step t + kSync - 1): every tile is read kSync
  // steps after its copy, so a barrier always lies between the two, and the
  // stage a copy overwrites was last read kSync steps before it.
  const TileDma<D, kWaves> dma;
  const uint8_t* const ktiles = a.kp + (size_t)bh * a.nblk * C::KT;
  const uint8_t* const vtiles = a.vp + (size_t)bh * a.nkb * C::VT;
  // smem is the kernel's only LDS variable, at LDS address 0 (the P-map
  // lookup relies on it): K stages follow the table, then the V stages.
  constexpr uint32_t kbase = kPTabBytes + kPThrBytes, vbase = kbase + kStages * C::KT;
  auto kst = [&](int t) { return opaque_s(kbase + (uint32_t)((t % kStages) * C::KT)); };
  auto vst = [&](int t) { return opaque_s(vbase + (uint32_t)((t % kStages) * C::VT)); };
  dma.issue(ktiles, nullptr, kst(0), vst(0));
  wait_lds_dma();
  __syncthreads();
#pragma unroll
  for (int i = 1; i <= kSync; ++i)
    dma.issue(i < nkb ? ktiles + i * C::KT : nullptr, i < kSync && i - 1 < nkb ? vtiles + (i - 1) * C::VT : nullptr,
              kst(i), vst(i - 1));
  v16f s[2];
  qk_step<D>(kst(0), qop, s);
  {
    const int nv0 = min(kBlock, a.N);
    if (nv0 < kBlock) mask_scores(s, nv0);
  }
  float cp_cur = score_scale(cq, sk[0], a.alpha);
  st.m = running_max(s, cp_cur, -INFINITY);
  wait_lds_dma();
  __syncthreads();
  // The key loop, with the K scales read through skp (LDS or global).
  const auto skp = [&]() {
    if constexpr (SKL) return (const float*)skl;
    else return sk;
  }();
  const uint8_t* ktn = ktiles + (kSync + 1) * C::KT;   // K tile of step t + kSync + 1
  const uint8_t* vtn = vtiles + (kSync - 1) * C::VT;   // V tile of step t + kSync - 1
  float m_prev = -INFINITY;                             // running max before step t
  uint32_t pp[2][4];                                    // codes of step t - 1
  // One step t < nkb - 1: P x V of step t - 1 (its MFMAs run under this
  // step's P-map work), the codes of step t, the rescale by
  // 2^(m(t-1) - m(t)) the accumulators need before P x V of step t, then S
  // and the running max of step t+1.  FIRST: t = 0; RAGGED: step t+1 may be
  // the last one.
  auto step = [&](int t, auto ragged, auto sync, auto first) {
    dma.issue(t + kSync + 1 < nkb ? ktn : nullptr, t + kSync - 1 < nkb ? vtn : nullptr, kst(t + kSync + 1),
              vst(t + kSync - 1));
    if constexpr (!decltype(first)::value) {
      pv_step<D>(vst(t - 1), pp, st.acc);
      lsum_step(lsum_selector_at_use(), pp, st.lsum);
    }
    uint32_t p[2][4];
    pmap_codes(s, cp_cur * kPIdxScale, st.m * kPIdxScale + 0.0f, a.pm.top_sub, ptab, p);
    if constexpr (DUMP) row_digest(p, t, dsum, dhash);
    if constexpr (!decltype(first)::value) {
      if (__ballot(st.m > m_prev) != 0) {
        const float beta = exp2f(m_prev - st.m);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) st.acc[dt][r] *= beta;
        st.lsum *= beta;
      }
    }
    qk_step<D>(kst(t + 1), qop, s);       // S of step t+1
    if constexpr (decltype(ragged)::value) {
      const int nv1 = a.N - (t + 1) * kBlock;
      if (nv1 < kBlock) mask_scores(s, opaque_sgpr(nv1));
    }
    const float cp_next = score_scale(cq, skp[t + 1], a.alpha);
    m_prev = st.m;
    st.m = running_max(s, cp_next, st.m);
    cp_cur = cp_next;
#pragma unroll
    for (int i = 0; i < 8; ++i) pp[i >> 2][i & 3] = p[i >> 2][i & 3];
    if constexpr (decltype(sync)::value) {
      wait_lds_dma();
      __syncthreads();
    }
    ktn += C::KT;
    vtn += C::VT;
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (nkb > 1) {
    // Barriers after the steps t with t % kSync == 0.
    step(0, T_{}, T_{}, T_{});
    int t0 = 1;
    // Whole blocks in which no step is followed by the last one.
#pragma nounroll
    for (; t0 + kSync + 1 < nkb; t0 += kSync) {
#pragma unroll
      for (int i = 0; i + 1 < kSync; ++i) step(t0 + i, F_{}, F_{}, F_{});
      step(t0 + kSync - 1, F_{}, T_{}, F_{});
    }
    // The remaining steps but the last, with a barrier after each.
#pragma nounroll
    for (; t0 + 1 < nkb; ++t0) step(t0, T_{}, T_{}, F_{});
    // The last step: P x V of step t - 1, the rescale, its codes, and its
    // own P x V after a barrier (its V tile was copied fewer than kSync
    // steps ago).
    const int t = nkb - 1, nvalid = a.N - t * kBlock;
    pv_step<D>(vst(t - 1), pp, st.acc);
    lsum_step(lsum_selector_at_use(), pp, st.lsum);
    uint32_t p[2][4];
    pmap_codes(s, cp_cur * kPIdxScale, st.m * kPIdxScale + 0.0f, a.pm.top_sub, ptab, p);
    if (nvalid < kBlock) mask_p(p, nvalid);
    if constexpr (DUMP) row_digest(p, t, dsum, dhash);
    if (__ballot(st.m > m_prev) != 0) {
      const float beta = exp2f(m_prev - st.m);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[dt][r] *= beta;
      st.lsum *= beta;
    }
    wait_lds_dma();
    __syncthreads();
    pv_step<D>(vst(t), p, st.acc);
    lsum_step(lsum_selector_at_use(), p, st.lsum);
  } else {
    // A single key step (N <= 64).
    uint32_t p[2][4];
    pmap_codes(s, cp_cur * kPIdxScale, st.m * kPIdxScale + 0.0f, a.pm.top_sub, ptab, p);
    if (a.N < kBlock) mask_p(p, a.N);
    if constexpr (DUMP) row_digest(p, 0, dsum, dhash);
    pv_step<D>(vst(0), p, st.acc);
    lsum_step(lsum_selector_at_use(), p, st.lsum);
  }

  if constexpr (DUMP) {
    dsum = xhalf_sum_u(dsum);
    dhash = xhalf_sum_u(dhash);
    const int q = q0 + ln;
    if (hf == 0 && q < a.N) {
      uint32_t* r = a.row_dbg + ((size_t)bh * a.N + q) * 4;
      *reinterpret_cast<uint4*>(r) = make_uint4(__float_as_uint(st.m), dsum, dhash, __float_as_uint(st.lsum[0]));
    }
  }

  // o = A s_v / L: the scale of the dequantized P cancels against the
  // quantized row sum.  With the V-side Hadamard the V codes are of V H, and
  // the row is multiplied by H again.
  const float inv = 1.0f / st.lsum[0];
  if (VH) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const v4f sv = *reinterpret_cast<const v4f*>(a.s_v + (size_t)bh * D + dt * 32 + 8 * g + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) st.acc[dt][4 * g + e] = st.acc[dt][4 * g + e] * sv[e] * inv;
      }
    fwht_out<D>(st.acc);
  }
  // The rows leave through LDS, one 32-channel tile at a time: each lane
  // holds 4-channel pieces of one query, so direct stores would write every
  // row in 32-byte pieces; staged, a store instruction writes whole 128-byte
  // row segments.  Each wave stages its 32 rows in its own LDS region (the
  // K/V stages, free once every wave has left the key loop).
  __syncthreads();
  constexpr uint32_t kRowB = 32 * 4 + 16;                   // staged row: 32 fp32 channels, padded
  const uint32_t obuf = (uint32_t)wave * 32u * kRowB;
  const int b = bh / a.H, h = bh % a.H;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = dt * 32 + 8 * g + 4 * hf;
      v4f o;
      if (VH) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = st.acc[dt][4 * g + e];
      } else {
        const v4f sv = *reinterpret_cast<const v4f*>(a.s_v + (size_t)bh * D + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = st.acc[dt][4 * g + e] * sv[e] * inv;
      }
      *reinterpret_cast<__attribute__((address_space(3))) v4f*>(obuf + ln * kRowB + (8 * g + 4 * hf) * 4) = o;
    }
    // Read back by the same wave (its LDS accesses stay in order): lane l
    // takes 16 bytes of row 8 i + l / 8.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3), c = lane & 7;
      const v4f o = *reinterpret_cast<const __attribute__((address_space(3))) v4f*>(obuf + r * kRowB + c * 16);
      const int q = q0 + r;
      if (q < a.N) {
        const size_t oe = (((size_t)b * a.N + q) * a.H + h) * D + dt * 32 + 4 * c;
        if (OUT_BF16) {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + oe) =
              make_uint2((uint32_t)f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16),
                         (uint32_t)f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16));
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + oe) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }
}

// Debug: the same per-step building blocks for the 64 queries of one Q
// block, in program order, dumping step kv_blk.  Two waves, one stage.
template <int D>
__global__ __launch_bounds__(128) void k_int4_tile_dump(AttnArgs a, TileDumpArgs t) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kPTabBytes + kPThrBytes + C::KT + C::VT];
  uint8_t* const ptab = smem;
  constexpr uint32_t tiles = kPTabBytes + kPThrBytes;      // LDS address of the K tile, then the V tile
  ptab_copy<2>(a.ptab, ptab);                               // visible after the first barrier
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  const int bh = t.bh;
  const int q0 = t.q_blk * kBlock + wave * 32;
  v8i qop[C::QC];
  load_q<D>(a, bh, q0 + ln, hf, qop);
  const float cq = a.s_q[(size_t)bh * a.nblk + t.q_blk];
  State<D> st;
  state_init<D>(st);
  const TileDma<D, 2> dma;
  for (int kb = 0; kb <= t.kv_blk; ++kb) {
    dma.issue(a.kp + ((size_t)bh * a.nblk + kb) * C::KT, a.vp + ((size_t)bh * a.nkb + kb) * C::VT, tiles,
              tiles + C::KT);
    wait_lds_dma();
    __syncthreads();
    const int nvalid = min(kBlock, a.N - kb * kBlock);
    const float sk = a.s_k[(size_t)bh * a.nblk + kb];
    if (kb == t.kv_blk)
      tile_step<D, true>(tiles, tiles + C::KT, ptab, qop, cq, a.alpha, sk, nvalid, st, &t, wave, a.pm.P, a.pm.top_sub);
    else
      tile_step<D, false>(tiles, tiles + C::KT, ptab, qop, cq, a.alpha, sk, nvalid, st, nullptr, wave, a.pm.P, a.pm.top_sub);
    __syncthreads();
  }
}

// The kernels' P map on exponents d: the same table, lookup, marked-cell
// decision and packing as a step of the attention, with S = d, c = 1 and
// m = 0 (so x = -d exactly).  Each lane maps 32 consecutive values, as a
// lane maps its 32 scores of a step; u = code + zero-point.
__global__ __launch_bounds__(256) void k_pmap_probe(const float* __restrict__ d, uint8_t* __restrict__ u,
                                                    int64_t n, PMapArgs pm, const uint8_t* ptab) {
  __shared__ __attribute__((aligned(16))) uint8_t tab[kPTabTotal];   // the kernel's only LDS: address 0
  ptab_copy<4>(ptab, tab);
  wait_lds_dma();
  __syncthreads();
  const int64_t groups = (n + 31) / 32;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < groups; g += stride) {
    const int64_t base = g * 32;
    v16f s[2];
#pragma unroll
    for (int k = 0; k < 32; ++k) s[k >> 4][k & 15] = base + k < n ? d[base + k] : 0.0f;
    uint32_t p[2][4];
    pmap_codes(s, kPIdxScale, 0.0f, pm.top_sub, tab, p);
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (base + k < n) u[base + k] = (uint8_t)e4m3_to_uint((p[k >> 4][(k & 15) >> 2] >> (8 * (k & 3))) & 0xFFu);
  }
}

__global__ void k_copy16(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n16) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) dst[i] = src[i];
}

__global__ void k_copy1(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

template <int D, bool VH, bool DUMP>
static void launch_attn_d(const AttnArgs& a, bool out_bf16, unsigned nwg, hipStream_t st) {
  const dim3 blk(64 * kWaves);
  if (a.nkb <= kSkLds) {
    if (out_bf16) k_int4_attn<D, true, VH, DUMP, true><<<nwg, blk, 0, st>>>(a);
    else k_int4_attn<D, false, VH, DUMP, true><<<nwg, blk, 0, st>>>(a);
  } else {
    if (out_bf16) k_int4_attn<D, true, VH, DUMP, false><<<nwg, blk, 0, st>>>(a);
    else k_int4_attn<D, false, VH, DUMP, false><<<nwg, blk, 0, st>>>(a);
  }
}

template <bool DUMP>
static void launch_attn(const AttnArgs& a, int D, bool out_bf16, int B, hipStream_t st) {
  const unsigned nwg = (unsigned)(B * a.H * ((a.N + kQTile - 1) / kQTile));
  const bool vh = a.v_hadamard != 0;
  if (D == 128) {
    if (vh) launch_attn_d<128, true, DUMP>(a, out_bf16, nwg, st);
    else launch_attn_d<128, false, DUMP>(a, out_bf16, nwg, st);
  } else {
    if (vh) launch_attn_d<64, true, DUMP>(a, out_bf16, nwg, st);
    else launch_attn_d<64, false, DUMP>(a, out_bf16, nwg, st);
  }
}

void launch_int4_attn(const AttnArgs& a, int D, bool out_bf16, int B, hipStream_t st) {
  launch_attn<false>(a, D, out_bf16, B, st);
}

void launch_int4_attn_rowdbg(const AttnArgs& a, int D, int B, hipStream_t st) {
  launch_attn<true>(a, D, false, B, st);
}

void launch_int4_tile_dump(const AttnArgs& a, const TileDumpArgs& t, int D, hipStream_t st) {
  if (D == 128) k_int4_tile_dump<128><<<1, 128, 0, st>>>(a, t);
  else k_int4_tile_dump<64><<<1, 128, 0, st>>>(a, t);
}

void launch_pmap_probe(const float* d, uint8_t* u, int64_t n, const PMapArgs& pm, const uint8_t* ptab,
                       hipStream_t st) {
  if (n <= 0) return;
  const int64_t blocks = ((n + 31) / 32 + 255) / 256;
  k_pmap_probe<<<(unsigned)(blocks < 2048 ? blocks : 2048), 256, 0, st>>>(d, u, n, pm, ptab);
}

void launch_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16) k_copy16<<<2048, 256, 0, st>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  const size_t rem = bytes - n16 * 16;
  if (rem) k_copy1<<<1, 256, 0, st>>>(static_cast<const uint8_t*>(src) + n16 * 16,
                                      static_cast<uint8_t*>(dst) + n16 * 16, rem);
}

}  // namespace ra
