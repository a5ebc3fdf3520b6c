// ra_prologue.hip -- prologue kernels: 3D RoPE + RoPE-aware rotation + INT4
// quantization of Q/K, per-channel INT4 quantization of V, and the bf16
// preparation used by the full-precision fallback.
//
// Method source: "RotateAttention: RoPE-Aware Rotation and Range Rectification
// for INT4 Quantized Attention in Video Generation" (pith.science review):
// Sec. 3 / Fig. 2 (frame/height/width RoPE segments), Sec. 4.1 / Fig. 3
// (Interleaved rotation merged into RoPE, Half rotation with H2 blocks),
// abstract (INT4 Q/K/V inside FlashAttention).  The 64-token Q/K scale block
// follows the FlashAttention-tile-aligned blocks of the PAROAttention review.
//
// All kernels are HBM-bound streaming passes; every workgroup reads a 64-token
// x D tile once (16-byte loads), does the arithmetic in fp32 registers/LDS and
// writes packed output with 16-byte stores.
#include <type_traits>

#include "ra_common.h"
#include "ra_kernels.h"

namespace ra {

template <bool BF16> struct InT;
template <> struct InT<true> { typedef uint16_t T; };
template <> struct InT<false> { typedef float T; };

// Load one token row segment of `cnt` elements (cnt*sizeof(T) a multiple of
// 16 bytes) starting at p into LDS row `dst` as fp32.
template <bool BF16>
__device__ __forceinline__ void load_row_part(const void* base, size_t elem_off, int cnt, float* dst) {
  if (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
    for (int i = 0; i < cnt / 8; ++i) {
      uint4 w = p[i];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[8 * i + 2 * e] = __uint_as_float(ws[e] << 16);
        dst[8 * i + 2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
    for (int i = 0; i < cnt / 4; ++i) {
      float4 w = p[i];
      dst[4 * i] = w.x; dst[4 * i + 1] = w.y; dst[4 * i + 2] = w.z; dst[4 * i + 3] = w.w;
    }
  }
}

// Lane layout of the Q/K prologue kernels: a wave takes one token row at a
// time (two rows when D = 64, lanes 0-31 and 32-63) and lane j holds RoPE
// pair j, channels (2j, 2j+1), which lies in one segment (segment offsets
// are even).  Loads of the row and of the segment tables are contiguous
// across the lanes of a segment.
template <int D>
struct PairLane {
  static constexpr int PAIRS = D / 2;
  static constexpr int RPI = 64 / PAIRS;   // rows per wave step
  int sub, j, s, jj, npair, off;           // row in the step, pair, segment, pair in segment, pairs in segment, channel offset
  const float2* csn;

  __device__ __forceinline__ explicit PairLane(const RopeTabs& t) {
    const int lane = threadIdx.x & 63;
    sub = RPI == 1 ? 0 : lane / PAIRS;      // with one row per step the row is wave-uniform
    j = RPI == 1 ? lane : lane % PAIRS;
    const int p1 = t.seg[0] >> 1, p2 = p1 + (t.seg[1] >> 1);
    s = (j >= p1) + (j >= p2);
    jj = j - (s == 0 ? 0 : (s == 1 ? p1 : p2));
    npair = t.seg[s] >> 1;
    off = t.off[s];
    csn = t.csn[s];
  }

  // RoPE of (x0, x1) at axis position pos of this lane's segment: each
  // product rounded, then the difference / sum.
  __device__ __forceinline__ void rope(int pos, float x0, float x1, float& y0, float& y1) const {
    const float2 cv = csn[pos * npair + jj];
    const float c = cv.x, sv = cv.y;
    const float ac = x0 * c, bs = x1 * sv;
    const float as = x0 * sv, bc = x1 * c;
    y0 = ac - bs;
    y1 = as + bc;
  }
};

// Token n -> (frame, height, width) with w fastest, advanced row by row.
struct GridPos {
  int f, h, w;
  __device__ __forceinline__ GridPos(int n, const RopeTabs& t) {
    const int hw = t.dims[1] * t.dims[2];
    f = n / hw;
    h = (n - f * hw) / t.dims[2];
    w = n - f * hw - h * t.dims[2];
  }
  // Advance by k <= 2 tokens: two conditional carries per axis suffice.
  __device__ __forceinline__ void advance(int k, const RopeTabs& t) {
    w += k;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool cw = w >= t.dims[2];
      w = cw ? w - t.dims[2] : w;
      h = cw ? h + 1 : h;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bool ch = h >= t.dims[1];
      h = ch ? h - t.dims[1] : h;
      f = ch ? f + 1 : f;
    }
  }
  __device__ __forceinline__ int axis(int s) const { return s == 0 ? f : (s == 1 ? h : w); }
};

// Two consecutive elements of a [B, N, H, D] row as fp32.
template <bool BF16>
__device__ __forceinline__ void load_pair(const void* base, size_t elem_off, float& x0, float& x1) {
  if (BF16) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + elem_off);
    x0 = __uint_as_float(w << 16);
    x1 = __uint_as_float(w & 0xFFFF0000u);
  } else {
    const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(base) + elem_off);
    x0 = v.x;
    x1 = v.y;
  }
}

__device__ __forceinline__ int quant_code(float x, float inv) {
  float q = __builtin_rintf(x * inv);
  q = fminf(fmaxf(q, -7.0f), 7.0f);
  return (int)q;
}

// Maximum of v over the 256 threads of the workgroup (red: 4 floats of LDS).
__device__ __forceinline__ float block_max_256(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  return m;
}

// Bits [32 W, 32 W + 32) of the 192-bit fp6 string of one (token, channel
// group): cw holds the group's 32 codes, one 6-bit code per byte.
template <int W>
__device__ __forceinline__ uint32_t fp6_word(const uint32_t (&cw)[8]) {
  constexpr int c_lo = 32 * W / 6;
  constexpr int c_hi = (32 * W + 31) / 6 < 31 ? (32 * W + 31) / 6 : 31;
  uint64_t acc = 0;
#pragma unroll
  for (int c = c_lo; c <= c_hi; ++c)
    acc |= (uint64_t)((cw[c >> 2] >> (8 * (c & 3))) & 0x3Fu) << (6 * (c - c_lo));
  return (uint32_t)(acc >> (32 * W - 6 * c_lo));
}

__device__ __forceinline__ void load_group_codes(const uint8_t* p, uint32_t (&cw)[8]) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
  cw[0] = a.x; cw[1] = a.y; cw[2] = a.z; cw[3] = a.w;
  cw[4] = b.x; cw[5] = b.y; cw[6] = b.z; cw[7] = b.w;
}

// Orthonormal Walsh-Hadamard transform (the full rotation of Q/K, and the
// V-side Hadamard of the RotateAttention review's summary) of a row of D
// values held VEC consecutive values per lane by
// D/VEC consecutive lanes.  Butterfly stages h = 1, 2, ..., D/2 in that
// order, each pair (i, i + h), bit h of i clear, becoming (x_i + x_{i+h},
// x_i - x_{i+h}): stages below VEC inside the lane, the others with the lane
// whose index differs in bit h / VEC; then one multiply by f32(1/sqrt(D)).
// Every lane of a row's group must execute it.
template <int VEC, int D>
__device__ __forceinline__ void fwht_row(float (&x)[VEC]) {
#pragma unroll
  for (int h = 1; h < VEC; h <<= 1)
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      if (!(i & h)) {
        const float lo = x[i], hi = x[i + h];
        x[i] = lo + hi;
        x[i + h] = lo - hi;
      }
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int h = VEC; h < D; h <<= 1) {
    const int m = h / VEC;
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float other = __shfl_xor(x[i], m, 64);
      x[i] = upper ? other - x[i] : x[i] + other;
    }
  }
  constexpr float sc = D == 128 ? 0.088388347648318440550f : 0.125f;   // f32(1/sqrt(D))
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
#pragma unroll
  for (int i = 0; i < VEC; ++i) x[i] = x[i] * sc;
}

// ---------------------------------------------------------------------------
// Q/K: one workgroup per (64-token block, b*h, tensor); each of the 4 waves
// takes 16 rows of the block (PairLane layout).  RoPE per pair, then (ROT ==
// 2) the Half rotation u' = (u + w) r, w' = (u - w) r on channels
// (i, i + L/2) of each segment through a per-wave LDS row, r = f32(1/sqrt 2);
// ROT == 1 (Interleaved) is already merged into the tables as +pi/4; ROT ==
// 3 (Full) multiplies the whole RoPE'd row by the Walsh-Hadamard matrix.  The
// rotated values stay in registers for the block amax, then become INT4
// codes held as fp16 values in an LDS tile; one conversion instruction per
// (token, 32-channel group) packs them into the fp6 e2m3 string of the
// 64-token tile, written with coalesced stores.  Eight waves
// per SIMD (64 registers, a few spilled): the loads of more blocks in flight
// outweigh the spills in this latency-bound pass.
template <int ROT, bool BF16, int D>
__global__ __launch_bounds__(256, 8) void k_rope_quant_qk(QKPrologueArgs a) {
  using PL = PairLane<D>;
  constexpr int ITERS = 16 / PL::RPI;
  __shared__ float red[4];
  // The block's codes as fp16 values (exact for -7..7), [row][channel],
  // rows padded by 16 bytes so that the 64-byte group reads spread over the
  // banks.
  constexpr int kCbRow = 2 * D + 16;
  __shared__ __attribute__((aligned(16))) uint8_t cb[kBlock * kCbRow];
  const int blk = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const int b = bh / a.H, h = bh % a.H;
  const void* x = which ? a.k : a.q;
  uint8_t* out = which ? a.k_out : a.q_out;
  float* sc = which ? a.s_k : a.s_q;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const PL pl(a.tabs);
  const int r0 = wave * 16 + pl.sub;
  GridPos gp(blk * kBlock + r0, a.tabs);

  // Pass 1: all rows' loads and RoPE, with no barrier in between, so every
  // load of the wave's 16 rows (inputs and table entries) is in flight at
  // once.
  // Blocks that lie wholly inside N (all but the ragged last one) skip the
  // per-row bounds check.
  float y[ITERS][2];
  const size_t row0 = ((size_t)b * a.N + (size_t)blk * kBlock + r0) * a.H + h;   // [B, N, H] row index
  auto pass1 = [&](auto check) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int n = blk * kBlock + r0 + it * PL::RPI;
      const bool ok = !decltype(check)::value || n < a.N;
      float x0 = 0.0f, x1 = 0.0f;
      if (ok) load_pair<BF16>(x, (row0 + (size_t)it * PL::RPI * a.H) * D + 2 * pl.j, x0, x1);
      pl.rope(ok ? gp.axis(pl.s) : 0, x0, x1, y[it][0], y[it][1]);
      gp.advance(PL::RPI, a.tabs);
    }
  };
  if ((blk + 1) * kBlock <= a.N) pass1(std::false_type{});
  else pass1(std::true_type{});
  // Pass 2 (Half): the partner of channel i of a segment, i +- L/2, is read
  // from the lane holding it with a cross-lane permute (no LDS allocation).
  // With L/2 even the partners of both channels of a pair sit at the same
  // element of one lane; with L/2 odd they sit at the other element of two
  // lanes.  Either way one permute of element 0 and one of element 1 fetch
  // both, and u' = (u + w) r, w' = (u - w) r become fma(own, +-1, other) r.
  if (ROT == 2) {
    const float r = __uint_as_float(0x3F3504F3u);
    const int hc = pl.npair;                 // L / 2 channels
    int src[2];
    float sgn[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * pl.jj + e;
      const bool first = i < hc;             // own is u, partner is w
      const int pi = first ? i + hc : i - hc;
      src[e] = pl.sub * PL::PAIRS + (pl.off >> 1) + (pi >> 1);
      sgn[e] = first ? 1.0f : -1.0f;
    }
    const bool odd = (hc & 1) != 0;
    const int sa = odd ? src[1] : src[0], sb = odd ? src[0] : src[1];   // element 0 from sa, 1 from sb
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const float pa = __shfl(y[it][0], sa, 64), pb = __shfl(y[it][1], sb, 64);
      const float o0 = odd ? pb : pa, o1 = odd ? pa : pb;
      y[it][0] = __builtin_fmaf(y[it][0], sgn[0], o0) * r;
      y[it][1] = __builtin_fmaf(y[it][1], sgn[1], o1) * r;
    }
  }
  // Full rotation: the whole RoPE'd row times the Walsh-Hadamard matrix; the
  // PAIRS lanes of a row hold it two values each.
  if (ROT == 3) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) fwht_row<2, D>(y[it]);
  }
  float mx = 0.0f;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) mx = fmaxf(mx, fmaxf(fabsf(y[it][0]), fabsf(y[it][1])));
  const float amax = block_max_256(mx, red);
  const float scale = amax / 7.0f;
  const float inv = 7.0f / amax;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int r = r0 + it * PL::RPI;
    // q = clamp(rint(x inv), -7, 7) (+ 0.0 turns -0 into +0); both codes of
    // the pair as fp16 (exact) in one 4-byte LDS word.
    const float q0 = amax > 0.0f ? __builtin_amdgcn_fmed3f(__builtin_rintf(y[it][0] * inv), -7.0f, 7.0f) + 0.0f : 0.0f;
    const float q1 = amax > 0.0f ? __builtin_amdgcn_fmed3f(__builtin_rintf(y[it][1] * inv), -7.0f, 7.0f) + 0.0f : 0.0f;
    *reinterpret_cast<uint32_t*>(cb + r * kCbRow + 4 * pl.j) =
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(q0, q1));
  }
  if (threadIdx.x == 0) sc[(size_t)bh * a.nblk + blk] = amax > 0.0f ? scale : 0.0f;
  __syncthreads();

  // One (row r, channel group g) per thread: its 32 codes become the 192-bit
  // fp6 e2m3 string (code i at bits 6i .. 6i+5) in one conversion
  // instruction; bits 0..127 go to byte (64 g + r) 16 of the tile, bits
  // 128..191 to byte (D / 32) 1024 + (64 g + r) 8.
  uint8_t* tile = out + ((size_t)bh * a.Npad + (size_t)blk * kBlock) * (qk6_tile_bytes(D) / kBlock);
  for (int u = threadIdx.x; u < 2 * D; u += 256) {
    const int r = u & 63, g = u >> 6;
    typedef __fp16 v32h __attribute__((ext_vector_type(32)));
    typedef uint32_t v6u __attribute__((ext_vector_type(6)));
    const uint4* src = reinterpret_cast<const uint4*>(cb + r * kCbRow + 64 * g);
    const uint4 c0 = src[0], c1 = src[1], c2 = src[2], c3 = src[3];
    const uint32_t cw[16] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w,
                             c2.x, c2.y, c2.z, c2.w, c3.x, c3.y, c3.z, c3.w};
    const v32h codes = __builtin_bit_cast(v32h, cw);
    const v6u w = __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(codes, 1.0f);
    *reinterpret_cast<uint4*>(tile + (64 * g + r) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint2*>(tile + (D / 32) * 1024 + (64 * g + r) * 8) = make_uint2(w[4], w[5]);
  }
}

// ---------------------------------------------------------------------------
// V per-channel amax over a chunk of tokens, merged with atomicMax on the
// float bit pattern (order-preserving for non-negative floats).
template <bool BF16, int D, bool VH>
__global__ __launch_bounds__(256) void k_v_amax(VAmaxArgs a) {
  typedef typename InT<BF16>::T T;
  constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte load
  constexpr int CG = D / VEC;              // threads per row
  constexpr int PH = 256 / CG;             // rows per iteration
  __shared__ float red[PH][D];
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int t = threadIdx.x, cg = t % CG, ph = t / CG;
  const int n0 = blockIdx.x * a.chunk;
  const int n1 = min(a.N, n0 + a.chunk);
  float m[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) m[e] = 0.0f;
  for (int n = n0 + ph; n < n1; n += PH) {
    float v[VEC];
    load_row_part<BF16>(a.v, (((size_t)b * a.N + n) * a.H + h) * D + cg * VEC, VEC, v);
    if (VH) fwht_row<VEC, D>(v);       // the CG lanes of row n share n
#pragma unroll
    for (int e = 0; e < VEC; ++e) m[e] = fmaxf(m[e], fabsf(v[e]));
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[ph][cg * VEC + e] = m[e];
  __syncthreads();
  for (int d = t; d < D; d += 256) {
    float mm = 0.0f;
    for (int p = 0; p < PH; ++p) mm = fmaxf(mm, red[p][d]);
    atomicMax(a.vamax + (size_t)bh * D + d, __float_as_uint(mm));
  }
}

__global__ void k_zero_u32(uint32_t* p, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// V quantization + transpose into the PV operand layout: one workgroup per
// (64-key block, b*h); thread (d, hf) packs the 32 codes lane half hf of
// the PV MFMA supplies for channel d into one fp6 string (v6_* layout).
template <bool BF16, int D, bool VH>
__global__ __launch_bounds__(256) void k_v_quant(VQuantArgs a) {
  constexpr int PER = D / 4;
  // bf16 inputs without the Hadamard are held in LDS as their bf16 bits
  // (exact, and half the LDS, so more workgroups fit on a CU); otherwise fp32.
  constexpr bool RAW = BF16 && !VH;
  typedef typename std::conditional<RAW, uint16_t, float>::type TT;
  __shared__ TT tile[64][D + 2];
  const int kb = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int t = threadIdx.x, r = t >> 2, qq = t & 3;
  const int n = kb * kBlock + r;
  if constexpr (RAW) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) +
                                                      (((size_t)b * a.N + (n < a.N ? n : 0)) * a.H + h) * D + qq * PER);
#pragma unroll
    for (int i = 0; i < PER / 8; ++i) {
      const uint4 w = n < a.N ? src[i] : make_uint4(0u, 0u, 0u, 0u);
      uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[r][qq * PER + 8 * i]);
      dst[0] = w.x; dst[1] = w.y; dst[2] = w.z; dst[3] = w.w;
    }
  } else {
    float tmp[PER];
    if (n < a.N) {
      load_row_part<BF16>(a.v, (((size_t)b * a.N + n) * a.H + h) * D + qq * PER, PER, tmp);
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) tmp[e] = 0.0f;
    }
    if (VH) fwht_row<PER, D>(tmp);       // lanes 4r .. 4r+3 hold row r (padded rows stay 0)
#pragma unroll
    for (int e = 0; e < PER; ++e) tile[r][qq * PER + e] = tmp[e];
  }
  __syncthreads();
  auto val = [&](int key, int d) -> float {
    if constexpr (RAW) return __uint_as_float((uint32_t)tile[key][d] << 16);
    else return tile[key][d];
  };

  if (t < 2 * D) {
    const int d = t >> 1, hf = t & 1;
    const float amax = __uint_as_float(a.vamax[(size_t)bh * D + d]);
    const float inv = 7.0f / amax;
    uint32_t cw[8];                    // the 32 codes, one e2m3 code per byte
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) {
      uint32_t acc = 0;
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int key = slot_key_pv(v6_slot(hf, 4 * q4 + bi));
        const int c = amax > 0.0f ? quant_code(val(key, d), inv) : 0;
        acc |= e2m3_of_code(c) << (8 * bi);
      }
      cw[q4] = acc;
    }
    uint8_t* dst = a.v_out + ((size_t)bh * a.nkb + kb) * v6_tile_bytes(D);
    *reinterpret_cast<uint4*>(dst + v6_lo_off(D, d, hf)) =
        make_uint4(fp6_word<0>(cw), fp6_word<1>(cw), fp6_word<2>(cw), fp6_word<3>(cw));
    *reinterpret_cast<uint2*>(dst + v6_hi_off(D, d, hf)) = make_uint2(fp6_word<4>(cw), fp6_word<5>(cw));
    if (kb == 0 && hf == 0) a.s_v[(size_t)bh * D + d] = amax > 0.0f ? amax / 7.0f : 0.0f;
  }
}

// ---------------------------------------------------------------------------
// bf16 fallback preparation: RoPE in fp32 (no rotation, no quantization),
// rounded to bf16; padded rows are zero.  Q as rows [b*h][Npad][D]; K in
// 64-key tiles of 16-byte chunks, chunk (c / 8, key) of a tile at byte
// (c / 8 * 64 + key) * 16 (channels 8 (c / 8) .. + 7 of that key), the order
// in which the attention kernel copies a tile into LDS and reads its MFMA
// operands.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_rope_bf16(QKPrologueArgs a) {
  using PL = PairLane<D>;
  constexpr int ITERS = 16 / PL::RPI;
  // K tile staged in LDS in its chunk order, each 64-chunk group padded by 16
  // bytes so that the 4-byte pair writes of a row spread over the banks.
  constexpr int GSTRIDE = 64 * 16 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t kt[(D / 8) * GSTRIDE];
  const int blk = blockIdx.x, bh = blockIdx.y, which = blockIdx.z;
  const int b = bh / a.H, h = bh % a.H;
  const void* x = which ? a.k : a.q;
  uint16_t* out = reinterpret_cast<uint16_t*>(which ? a.k_out : a.q_out);
  const int wave = threadIdx.x >> 6;
  const PL pl(a.tabs);
  const int r0 = wave * 16 + pl.sub;
  GridPos gp(blk * kBlock + r0, a.tabs);
  const size_t row0 = ((size_t)b * a.N + (size_t)blk * kBlock + r0) * a.H + h;   // [B, N, H] row index
  // As in k_rope_quant_qk: no per-row bounds check on whole blocks.
  auto rows = [&](auto check) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int r = r0 + it * PL::RPI;
      const int n = blk * kBlock + r;
      const bool ok = !decltype(check)::value || n < a.N;
      float x0 = 0.0f, x1 = 0.0f;
      if (ok) load_pair<BF16>(x, (row0 + (size_t)it * PL::RPI * a.H) * D + 2 * pl.j, x0, x1);
      float v0, v1;
      pl.rope(ok ? gp.axis(pl.s) : 0, x0, x1, v0, v1);
      const uint32_t w = (uint32_t)f32_to_bf16_bits(v0) | ((uint32_t)f32_to_bf16_bits(v1) << 16);
      if (which)
        *reinterpret_cast<uint32_t*>(kt + (2 * pl.j / 8) * GSTRIDE + r * 16 + (2 * pl.j % 8) * 2) = w;
      else
        *reinterpret_cast<uint32_t*>(out + ((size_t)bh * a.Npad + blk * kBlock + r) * D + 2 * pl.j) = w;
      gp.advance(PL::RPI, a.tabs);
    }
  };
  if ((blk + 1) * kBlock <= a.N) rows(std::false_type{});
  else rows(std::true_type{});
  if (which) {
    __syncthreads();
    // 16-byte unit u of the tile = chunk (u / 64, u % 64), at byte 16 u.
    uint8_t* tile = reinterpret_cast<uint8_t*>(out + ((size_t)bh * a.Npad + (size_t)blk * kBlock) * D);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int u = threadIdx.x + 256 * i;
      *reinterpret_cast<uint4*>(tile + 16 * u) = *reinterpret_cast<const uint4*>(kt + (u >> 6) * GSTRIDE + (u & 63) * 16);
    }
  }
}

// V for the bf16 path: per 64-key block, 16-byte chunks (slot group g,
// channel d) at byte (g D + d) * 16, each the 8 keys of slots 8g .. 8g + 7 in
// the bf16 PV operand slot order; padded keys are zero.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void k_v_bf16(VQuantArgs a) {
  constexpr int PER = D / 4;
  __shared__ float tile[64][D + 1];
  const int kb = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int t = threadIdx.x, r = t >> 2, qq = t & 3;
  const int n = kb * kBlock + r;
  float tmp[PER];
  if (n < a.N) {
    load_row_part<BF16>(a.v, (((size_t)b * a.N + n) * a.H + h) * D + qq * PER, PER, tmp);
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) tmp[e] = 0.0f;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) tile[r][qq * PER + e] = tmp[e];
  __syncthreads();
  uint16_t* outp = reinterpret_cast<uint16_t*>(a.v_out);
  constexpr int UNITS = D * 8 / 256;       // (channel, 8-slot group) units per thread
#pragma unroll
  for (int uu = 0; uu < UNITS; ++uu) {
    const int unit = t * UNITS + uu;
    const int d = unit >> 3, g = unit & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x0 = tile[slot_key_bf16(g * 8 + 2 * e)][d];
      float x1 = tile[slot_key_bf16(g * 8 + 2 * e + 1)][d];
      w[e] = (uint32_t)f32_to_bf16_bits(x0) | ((uint32_t)f32_to_bf16_bits(x1) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(outp + ((size_t)bh * a.nkb + kb) * D * 64 + (g * D + d) * 8);
    *dst = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
#define RA_DISPATCH_D(D_, ...)                      \
  do {                                              \
    if ((D_) == 128) { constexpr int D = 128; __VA_ARGS__; } \
    else { constexpr int D = 64; __VA_ARGS__; }     \
  } while (0)

void launch_int4_prologue(const QKPrologueArgs& qa, const VAmaxArgs& va, const VQuantArgs& vq,
                          int D, int rot, bool in_bf16, bool vh, hipStream_t st) {
  const int BH = qa.B * qa.H;
  {
    size_t n = (size_t)BH * D;
    k_zero_u32<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(va.vamax, n);
  }
  dim3 gq(qa.nblk, BH, 2);
  RA_DISPATCH_D(D, {
    if (in_bf16) {
      if (rot == 0) k_rope_quant_qk<0, true, D><<<gq, 256, 0, st>>>(qa);
      else if (rot == 1) k_rope_quant_qk<1, true, D><<<gq, 256, 0, st>>>(qa);
      else if (rot == 2) k_rope_quant_qk<2, true, D><<<gq, 256, 0, st>>>(qa);
      else k_rope_quant_qk<3, true, D><<<gq, 256, 0, st>>>(qa);
      if (vh) {
        k_v_amax<true, D, true><<<dim3((va.N + va.chunk - 1) / va.chunk, BH), 256, 0, st>>>(va);
        k_v_quant<true, D, true><<<dim3(vq.nkb, BH), 256, 0, st>>>(vq);
      } else {
        k_v_amax<true, D, false><<<dim3((va.N + va.chunk - 1) / va.chunk, BH), 256, 0, st>>>(va);
        k_v_quant<true, D, false><<<dim3(vq.nkb, BH), 256, 0, st>>>(vq);
      }
    } else {
      if (rot == 0) k_rope_quant_qk<0, false, D><<<gq, 256, 0, st>>>(qa);
      else if (rot == 1) k_rope_quant_qk<1, false, D><<<gq, 256, 0, st>>>(qa);
      else if (rot == 2) k_rope_quant_qk<2, false, D><<<gq, 256, 0, st>>>(qa);
      else k_rope_quant_qk<3, false, D><<<gq, 256, 0, st>>>(qa);
      if (vh) {
        k_v_amax<false, D, true><<<dim3((va.N + va.chunk - 1) / va.chunk, BH), 256, 0, st>>>(va);
        k_v_quant<false, D, true><<<dim3(vq.nkb, BH), 256, 0, st>>>(vq);
      } else {
        k_v_amax<false, D, false><<<dim3((va.N + va.chunk - 1) / va.chunk, BH), 256, 0, st>>>(va);
        k_v_quant<false, D, false><<<dim3(vq.nkb, BH), 256, 0, st>>>(vq);
      }
    }
  });
}

void launch_bf16_prologue(const QKPrologueArgs& qa, const VQuantArgs& vq, int D, bool in_bf16,
                          hipStream_t st) {
  const int BH = qa.B * qa.H;
  dim3 gq(qa.nblk, BH, 2);
  RA_DISPATCH_D(D, {
    if (in_bf16) {
      k_rope_bf16<true, D><<<gq, 256, 0, st>>>(qa);
      k_v_bf16<true, D><<<dim3(vq.nkb, BH), 256, 0, st>>>(vq);
    } else {
      k_rope_bf16<false, D><<<gq, 256, 0, st>>>(qa);
      k_v_bf16<false, D><<<dim3(vq.nkb, BH), 256, 0, st>>>(vq);
    }
  });
}

}  // namespace ra
