// ra_bf16_attn.hip -- bf16 FlashAttention forward: the full-precision fallback
// used on the accuracy-sensitive denoising steps and DiT blocks.
//
// Method source: "RotateAttention: RoPE-Aware Rotation and Range Rectification
// for INT4 Quantized Attention in Video Generation" (pith.science review),
// Sec. 5.1: FP16 attention on the first/last sampling steps and DiT blocks.
// On gfx950 the fallback runs in bf16: RoPE'd Q/K and V in bf16, scores and
// softmax in fp32, P rounded to bf16 for PV, fp32 accumulation.
//
// Design (gfx950):
//   * 8 waves x 32 queries per workgroup; S^T = K Q^T in the accumulators of
//     v_mfma_f32_32x32x16_bf16, so each lane owns one query and its P values
//     are exactly the bytes it supplies as the B operand of PV.
//   * K and V tiles (16 KB each at D = 128) are laid out by the prologue in
//     16-byte operand chunks, K chunk (c / 8, key) and V chunk (slot group,
//     channel), so that a tile is copied from global memory into LDS as it
//     lies (LDS-direct buffer loads, no registers) and every operand read of
//     a wave is 64 consecutive chunks (no bank conflicts).
//   * 4 LDS stages of K and of V, a workgroup barrier every 2 steps.
//   * S is double-buffered: the QK MFMAs of step t+1 are issued before the
//     softmax of step t, whose exp2 work then runs while they execute; the
//     PV MFMAs of step t overlap the running max of step t+1.
#include <type_traits>

#include "ra_common.h"
#include "ra_kernels.h"

namespace ra {

namespace {

constexpr int kBWaves = 8;                 // waves per workgroup (32 queries each)
constexpr int kBSync = 2;                  // steps per workgroup barrier
constexpr int kBStages = 2 * kBSync;       // LDS stages of K and of V tiles

template <int D>
struct BCfg {
  static constexpr int KS = D / 16;        // 16-channel K-steps of Q.K
  static constexpr int DT = D / 32;        // 32-channel tiles of O
  static constexpr int KT = 64 * D * 2;    // bf16 K tile of 64 keys
  static constexpr int VT = 64 * D * 2;    // bf16 V tile of 64 keys
};

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const uint8_t blds_cu8;

__device__ __forceinline__ blds_cu8* blds(uint32_t a) { return (blds_cu8*)a; }

// A stage address the optimizer cannot see through (one scalar add per base
// instead of one register per read).
__device__ __forceinline__ uint32_t bopaque(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// 16-byte buffer load with the LDS-direct bit (as in the INT4 kernel): lane i
// copies 16 bytes from base(rsrc) + voffset into LDS at lds + 16 i.  Not
// modelled by the compiler as an LDS store; completion is ordered by
// bwait_dma() and the workgroup barrier.
__device__ __forceinline__ void bcopy16(v4i rsrc, uint32_t lds, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(rsrc)
               : "memory");
}
__device__ __forceinline__ void bwait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ v4i brsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
             __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)), (int)bytes, 0x00020000};
}

// One step's K and V tiles by the 8 waves: 2 x KT / 16 slots of 16 bytes,
// 64 consecutive slots per wave and instruction, K slots first.
template <int D>
struct BTileDma {
  static constexpr int KSL = BCfg<D>::KT / 16;
  static constexpr int NI = 2 * KSL / (64 * kBWaves);
  static_assert(KSL % (64 * kBWaves) == 0, "tiles must be whole workgroups of slots");
  int off;        // this lane's byte offset within its 64-slot run
  int wbase;      // the wave's first slot within an instruction's 512
  __device__ __forceinline__ BTileDma() {
    wbase = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * 64;
    off = (wbase + (int)(threadIdx.x & 63)) * 16;
  }
  __device__ __forceinline__ void issue(const uint8_t* kt, const uint8_t* vt, uint32_t kst, uint32_t vst) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      constexpr int half = NI / 2;
      const int first = (j % half) * 64 * kBWaves;          // slot of this instruction within its tile
      if (j < half) {
        if (kt != nullptr) bcopy16(brsrc(kt, BCfg<D>::KT), kst + (uint32_t)((first + wbase) * 16), off + first * 16);
      } else {
        if (vt != nullptr) bcopy16(brsrc(vt, BCfg<D>::VT), vst + (uint32_t)((first + wbase) * 16), off + first * 16);
      }
    }
  }
};

// S^T of one 64-key step: M-tile mt = keys 32 mt .. 32 mt + 31.  K chunk
// (c / 8, key) of the stage at byte (c / 8 * 64 + key) * 16.
template <int D>
__device__ __forceinline__ void bqk(uint32_t kst, const v8bf (&qop)[BCfg<D>::KS], v16f (&s)[2]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  blds_cu8* const kb = blds(kst + (uint32_t)((hf * 64 + ln) * 16));
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mt][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < BCfg<D>::KS; ++ks) {
      const v8bf ka = *reinterpret_cast<const __attribute__((address_space(3))) v8bf*>(kb + ks * 2048 + mt * 512);
      s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[ks], s[mt], 0, 0, 0);
    }
  }
}

// O^T += V^T P^T over the step.  V chunk (slot group g, channel) at byte
// (g D + channel) * 16; K-step ks of PV uses slot groups 2 ks + hf.
template <int D>
__device__ __forceinline__ void bpv(uint32_t vst, const v8bf (&pb)[4], v16f (&acc)[BCfg<D>::DT]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  blds_cu8* const vb = blds(vst + (uint32_t)((hf * D + ln) * 16));
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int dt = 0; dt < BCfg<D>::DT; ++dt) {
      const v8bf va = *reinterpret_cast<const __attribute__((address_space(3))) v8bf*>(vb + ks * 2 * D * 16 + dt * 512);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], acc[dt], 0, 0, 0);
    }
}

// Keys at or past nvalid get S = -inf (p = 0).
__device__ __forceinline__ void bmask(v16f (&s)[2], int nvalid) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (mt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3) >= nvalid) s[mt][r] = -INFINITY;
}

__device__ __forceinline__ int bopaque_i(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

// Running max (log2 units) of this lane's query after the step.
__device__ __forceinline__ float bmax(const v16f (&s)[2], float alpha, float m) {
  float mx = s[0][0];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
  mx = xhalf_max_f(mx);
  return fmaxf(m, mx * alpha);
}

// p = 2^(s alpha - m) rounded to bf16 in PV B-operand order (K-step ks of
// PV takes registers 8 (ks % 2) .. + 7 of M-tile ks / 2), and the row sum of
// the fp32 p.
__device__ __forceinline__ void bsoftmax(const v16f (&s)[2], float alpha, float m, v8bf (&pb)[4], float& l) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    v2bf h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r0 = 8 * (ks & 1) + 2 * e;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ks >> 1][r0], alpha, -m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ks >> 1][r0 + 1], alpha, -m));
      l += p0;
      l += p1;
      h[e] = __builtin_convertvector((v2f){p0, p1}, v2bf);
    }
    pb[ks] = (v8bf){h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
  }
}

}  // namespace

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(64 * kBWaves, 1) void k_bf16_attn(AttnArgs a) {
  using C = BCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kBStages * (C::KT + C::VT)];

  const int nwg = gridDim.x, wg = blockIdx.x;
  const int full = nwg & ~7;
  const int lid = wg < full ? (wg & 7) * (full >> 3) + (wg >> 3) : wg;
  const int bh = lid / a.nqt, qt = lid % a.nqt;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  const int q0 = qt * 256 + wave * 32;
  const int nkb = a.nkb;

  // Q operands: query q0+ln, channels 16ks + 8hf + 0..7 (rows [bh][Npad][D]).
  v8bf qop[C::KS];
  {
    const int q = q0 + ln;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (q < a.Npad)
        w = *reinterpret_cast<const uint4*>(a.qp + (((size_t)bh * a.Npad + q) * D + ks * 16 + hf * 8) * 2);
      qop[ks] = __builtin_bit_cast(v8bf, w);
    }
  }

  v16f acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
  float l = 0.0f;
  const float alpha = a.alpha;

  // Step t reads the K tile of step t+1 and the V tile of step t and issues
  // the copies of K of step t + kBSync + 1 and V of step t + kBSync; both are
  // first read kBSync steps later, after the barrier that follows the wait
  // for them, and the stages they overwrite were last read before the
  // barrier that precedes the copies.
  const BTileDma<D> dma;
  const uint8_t* const ktiles = a.kp + (size_t)bh * a.Npad * D * 2;
  const uint8_t* const vtiles = a.vp + (size_t)bh * a.nkb * C::VT;
  // LDS address of the stages (smem is referenced through its address, which
  // also keeps its allocation: every access goes through computed addresses).
  const uint32_t kbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const uint32_t vbase = kbase + kBStages * C::KT;
  auto kst = [&](int t) { return bopaque(kbase + (uint32_t)((t % kBStages) * C::KT)); };
  auto vst = [&](int t) { return bopaque(vbase + (uint32_t)((t % kBStages) * C::VT)); };
  dma.issue(ktiles, nullptr, kst(0), vst(0));
  bwait_dma();
  __syncthreads();
#pragma unroll
  for (int i = 1; i <= kBSync; ++i)
    dma.issue(i < nkb ? ktiles + i * C::KT : nullptr, i - 1 < nkb ? vtiles + (i - 1) * C::VT : nullptr, kst(i),
              vst(i - 1));
  v16f sa[2], sb[2];
  bqk<D>(kst(0), qop, sa);
  if (a.N < kBlock) bmask(sa, a.N);
  float m = bmax(sa, alpha, -INFINITY);
  bwait_dma();
  __syncthreads();
  const uint8_t* ktn = ktiles + (kBSync + 1) * C::KT;
  const uint8_t* vtn = vtiles + kBSync * C::VT;

  // Step t < nkb - 1 with S of step t in sc; S of step t+1 goes to sn.
  // RAGGED: step t+1 may be the last one, with N ending inside it; SYNC: the
  // barrier after this step.
  auto step = [&](int t, v16f(&sc)[2], v16f(&sn)[2], auto ragged, auto sync) {
    dma.issue(t + kBSync + 1 < nkb ? ktn : nullptr, t + kBSync < nkb ? vtn : nullptr, kst(t + kBSync + 1),
              vst(t + kBSync));
    bqk<D>(kst(t + 1), qop, sn);
    v8bf pb[4];
    bsoftmax(sc, alpha, m, pb, l);
    if constexpr (decltype(ragged)::value) {
      const int nv1 = a.N - (t + 1) * kBlock;
      if (nv1 < kBlock) bmask(sn, bopaque_i(nv1));
    }
    bpv<D>(vst(t), pb, acc);
    const float m_new = bmax(sn, alpha, m);
    if (__ballot(m_new > m) != 0) {
      const float beta = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= beta;
      l *= beta;
    }
    m = m_new;
    if constexpr (decltype(sync)::value) {
      bwait_dma();
      __syncthreads();
    }
    ktn += C::KT;
    vtn += C::VT;
  };
  // The last step: its V tile was copied at least kBSync steps ago.
  auto last = [&](int t, v16f(&sc)[2]) {
    v8bf pb[4];
    bsoftmax(sc, alpha, m, pb, l);
    bpv<D>(vst(t), pb, acc);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int t = 0;
  // Pairs of steps (t even: S of step t in sa) whose successors are not the
  // last step; the barrier after each odd step.
#pragma nounroll
  for (; t + 3 < nkb; t += 2) {
    step(t, sa, sb, F_{}, F_{});
    step(t + 1, sb, sa, F_{}, T_{});
  }
  if (t + 2 < nkb) {                       // t = nkb - 3
    step(t, sa, sb, F_{}, F_{});
    step(t + 1, sb, sa, T_{}, T_{});
    last(t + 2, sa);
  } else if (t + 1 < nkb) {                // t = nkb - 2
    step(t, sa, sb, T_{}, F_{});
    last(t + 1, sb);
  } else {                                 // t = nkb - 1
    last(t, sa);
  }

  const float lt = xhalf_sum_f(l);
  const float inv = 1.0f / lt;
  const int q = q0 + ln;
  if (q < a.N) {
    const int b = bh / a.H, h = bh % a.H;
    const size_t obase = (((size_t)b * a.N + q) * a.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = dt * 32 + 8 * g + 4 * hf;
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[dt][4 * g + e] * inv;
        if (OUT_BF16) {
          uint16_t* op = static_cast<uint16_t*>(a.out) + obase + d;
          *reinterpret_cast<uint2*>(op) =
              make_uint2((uint32_t)f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16),
                         (uint32_t)f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16));
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase + d) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
  }
}

void launch_bf16_attn(const AttnArgs& a, int D, bool out_bf16, int B, hipStream_t st) {
  const unsigned nwg = (unsigned)(B * a.H * a.nqt);
  const dim3 blk(64 * kBWaves);
  if (D == 128) {
    if (out_bf16) k_bf16_attn<128, true><<<nwg, blk, 0, st>>>(a);
    else k_bf16_attn<128, false><<<nwg, blk, 0, st>>>(a);
  } else {
    if (out_bf16) k_bf16_attn<64, true><<<nwg, blk, 0, st>>>(a);
    else k_bf16_attn<64, false><<<nwg, blk, 0, st>>>(a);
  }
}

}  // namespace ra
