// ra_bf16_attn.hip -- bf16 FlashAttention forward: the full-precision fallback
// used on the accuracy-sensitive denoising steps and DiT blocks.
//
// Method source: "RotateAttention: RoPE-Aware Rotation and Range Rectification
// for INT4 Quantized Attention in Video Generation" (pith.science review),
// Sec. 5.1: FP16 attention on the first/last sampling steps and DiT blocks.
// On gfx950 the fallback runs in bf16: RoPE'd Q/K and V in bf16, scores and
// softmax in fp32, P rounded to bf16 for PV, fp32 accumulation.
//
// Same tiling as the INT4 kernel (8 waves x 32 queries, 64-key steps, S^T in
// the accumulators so that P feeds PV without shuffles), on
// v_mfma_f32_32x32x16_bf16.  The output accumulator is rescaled only when some
// row's running max rises.
#include "ra_common.h"
#include "ra_kernels.h"

namespace ra {

template <int D>
struct BCfg {
  static constexpr int KS = D / 16;          // 16-channel K-steps of Q.K
  static constexpr int DT = D / 32;          // 32-channel tiles of O
  static constexpr int KROW = D * 2 + 16;    // LDS bytes per key row
  static constexpr int VROW = 64 * 2 + 16;   // LDS bytes per channel row
  static constexpr int KT = 64 * KROW;
  static constexpr int VT = D * VROW;
  static constexpr int STAGE = KT + VT;
  static constexpr int KPARTS = D / 8;       // 16-byte parts per key row
  static constexpr int KP = 64 * KPARTS;
  static constexpr int TOT = KP + 8 * D;     // + 8 parts per channel row of V
};

template <int D, int NT>
struct BTileLoad {
  static constexpr int NP = (BCfg<D>::TOT + NT - 1) / NT;
  static constexpr bool EXACT = BCfg<D>::TOT % NT == 0;
  v4u r[NP];
  __device__ __forceinline__ void fetch(const AttnArgs& a, int bh, int kb) {
    using C = BCfg<D>;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = threadIdx.x + i * NT;
      const int pv = p - C::KP;
      const bool isk = (C::KP % NT == 0) ? (i * NT < C::KP) : (p < C::KP);
      const uint8_t* src = isk
          ? a.kp + (((size_t)bh * a.Npad + (size_t)kb * kBlock + p / C::KPARTS) * D + (p % C::KPARTS) * 8) * 2
          : a.vp + ((((size_t)bh * a.nkb + kb) * D + (pv >> 3)) * 64 + (pv & 7) * 8) * 2;
      if (EXACT || p < C::TOT) r[i] = *reinterpret_cast<const v4u*>(src);
    }
  }
  __device__ __forceinline__ void store(uint8_t* stage) const {
    using C = BCfg<D>;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = threadIdx.x + i * NT;
      if (!EXACT && p >= C::TOT) continue;
      const int pv = p - C::KP;
      const bool isk = (C::KP % NT == 0) ? (i * NT < C::KP) : (p < C::KP);
      const int o = isk ? (p / C::KPARTS) * C::KROW + (p % C::KPARTS) * 16
                              : C::KT + (pv >> 3) * C::VROW + (pv & 7) * 16;
      *reinterpret_cast<v4u*>(stage + o) = r[i];
    }
  }
};

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(512) void k_bf16_attn(AttnArgs a) {
  using C = BCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int nwg = gridDim.x, wg = blockIdx.x;
  const int full = nwg & ~7;
  const int lid = wg < full ? (wg & 7) * (full >> 3) + (wg >> 3) : wg;
  const int bh = lid / a.nqt, qt = lid % a.nqt;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  const int q0 = qt * 256 + wave * 32;

  // Q operands: query q0+ln, channels 16ks + 8hf + 0..7.
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
  float m = -INFINITY, l = 0.0f;
  const float alpha = a.alpha;

  BTileLoad<D, 512> ld;
  ld.fetch(a, bh, 0);
  ld.store(smem);
  __syncthreads();
  for (int kb = 0; kb < a.nkb; ++kb) {
    const bool more = kb + 1 < a.nkb;
    if (more) ld.fetch(a, bh, kb + 1);
    const uint8_t* stage = smem + (kb & 1) * C::STAGE;
    const int nvalid = min(kBlock, a.N - kb * kBlock);

    v16f s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mt][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const v8bf ka = *reinterpret_cast<const v8bf*>(stage + (mt * 32 + ln) * C::KROW + ks * 32 + hf * 16);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[ks], s[mt], 0, 0, 0);
      }
    }
    if (nvalid < kBlock) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3) >= nvalid) s[mt][r] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
    mx = xhalf_max_f(mx);
    const float m_new = fmaxf(m, mx * alpha);
    if (__ballot(m_new > m) != 0) {
      const float beta = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= beta;
      l *= beta;
    }
    m = m_new;

    // p = 2^(s alpha - m); K-step ks of PV takes registers 8(ks%2)..+7 of M-tile ks/2.
    v8bf pb[4];
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
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const v8bf va = *reinterpret_cast<const v8bf*>(stage + C::KT + (dt * 32 + ln) * C::VROW + ks * 32 + hf * 16);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], acc[dt], 0, 0, 0);
      }
    if (more) ld.store(smem + ((kb + 1) & 1) * C::STAGE);
    __syncthreads();
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
  if (D == 128) {
    if (out_bf16) k_bf16_attn<128, true><<<nwg, 512, 0, st>>>(a);
    else k_bf16_attn<128, false><<<nwg, 512, 0, st>>>(a);
  } else {
    if (out_bf16) k_bf16_attn<64, true><<<nwg, 512, 0, st>>>(a);
    else k_bf16_attn<64, false><<<nwg, 512, 0, st>>>(a);
  }
}

}  // namespace ra
