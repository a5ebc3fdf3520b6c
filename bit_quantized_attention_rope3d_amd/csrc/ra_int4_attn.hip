// ra_int4_attn.hip -- INT4 FlashAttention forward with range-optimized P.
//
// Method source: "RotateAttention: RoPE-Aware Rotation and Range Rectification
// for INT4 Quantized Attention in Video Generation" (pith.science review):
// abstract (INT4 Q, K, V inside FlashAttention; P = exp(QK - max QK)) and
// Sec. 4.2 (P mapped onto the full signed INT4 range: code = round(15 p) - 8).
//
// gfx950 design
//   * One workgroup = 8 waves = 256 query rows of one (b, h); each wave owns 32
//     queries.  Workgroup ids are remapped so that the workgroups resident on
//     one XCD walk the same head, sharing K/V tiles in that XCD's L2.
//   * Per 64-key step the packed INT4 K and V tiles (4 KB + 4 KB for D = 128)
//     are fetched with one 16-byte load per thread, widened once per
//     workgroup to int8 (x16, a shift and two masks per 8 codes) into LDS
//     (XOR-swizzled rows, no padding), double-buffered, one barrier per step.
//   * S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 with the INT4 codes widened to
//     fp8 e4m3 (exact for |code| <= 7; every partial sum is an integer below
//     2^24, so the fp32 accumulator holds the exact integer score and no
//     int->float conversion is needed).  Each lane holds one query column, so
//     row max / row sum are in-lane (+1 cross-half swap).
//   * P codes come straight out of the accumulator registers as bytes
//     (exponent FMA, round, exp2, cvt_pk_u8) in the order the PV MFMA wants
//     them as its B operand; V is stored pre-permuted to match.
//   * PV accumulates u * vhat in INT32 registers across steps; the fp32
//     accumulator lives in LDS (16 KB per wave) and is touched only when some
//     row's running max rises (then A = (A + I) * beta), which is rare after
//     the first few steps.  This keeps a wave within 256 VGPRs, i.e. two
//     waves per SIMD.
#include "ra_common.h"
#include "ra_kernels.h"

namespace ra {

template <int D>
struct Cfg {
  static constexpr int QC = D / 64;        // 64-channel chunks of the Q.K contraction
  static constexpr int DT = D / 32;        // 32-channel tiles of O
  static constexpr int KT = 64 * D;        // fp8 K tile: 64 rows of D bytes
  static constexpr int VT = D * 64;        // int8 V tile: D rows of 64 slots
  static constexpr int KPARTS = D / 32;    // 16-byte packed parts per key row
  static constexpr int KP = 64 * KPARTS;   // packed K parts per tile
  static constexpr int TOT = KP + 2 * D;   // + packed V parts (2 per channel)
  static constexpr int ACCF = DT * 4 * 64 * 16;   // LDS bytes of one wave's fp32 accumulator
};

// LDS rows are XOR-swizzled in 16-byte chunks.  The gfx950 LDS serves a
// ds_read_b128 / ds_write_b128 in groups of 16 lanes over 64 banks (256 B);
// the operand reads of one group touch 16 consecutive rows at one logical
// chunk, so the swizzle must give those 16 rows 16 distinct 16-byte slots
// of the 256-byte bank window: row parity (128-byte rows) or row mod 4
// (64-byte rows) picks the half / quarter, the XOR picks the slot within it.
template <int ROWBYTES>
__device__ __forceinline__ int swz(int row, int chunk) {
  if (ROWBYTES == 128) return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
  return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

template <int D>
struct State {
  v16i acc_i[Cfg<D>::DT];   // INT32 sum of u * (16 vhat) since the last rescale
  float m;                  // running max (grid units), this lane's query
  float L;                  // fp32 part of the row sum
  uint32_t U;               // integer row sum of u since the last rescale (lane half)
  float* accf;              // this wave's fp32 accumulator in LDS: [DT*4][64 lanes][4]
};

// Cooperative fetch of packed tiles into registers and widening store into
// LDS.  The K part and the V part may belong to different key steps (the
// pipelined main loop keeps K one step ahead of V); a negative index skips it.
template <int D, int NT>
struct TileLoad {
  static constexpr int NP = (Cfg<D>::TOT + NT - 1) / NT;
  static constexpr bool EXACT = Cfg<D>::TOT % NT == 0;
  v4u r[NP];

  __device__ __forceinline__ void fetch(const AttnArgs& a, int bh, int kt, int vt) {
    using C = Cfg<D>;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = threadIdx.x + i * NT;
      const int pv = p - C::KP;
      const bool isk = p < C::KP;
      const int t = isk ? kt : vt;
      const uint8_t* src = isk
          ? a.kp + ((size_t)bh * a.Npad + (size_t)kt * kBlock + p / C::KPARTS) * (D / 2) + (p % C::KPARTS) * 16
          : a.vp + (((size_t)bh * a.nkb + vt) * D + (pv >> 1)) * 32 + (pv & 1) * 16;
      if ((EXACT || p < C::TOT) && t >= 0) r[i] = *reinterpret_cast<const v4u*>(src);
    }
  }

  __device__ __forceinline__ void store(uint8_t* kst, uint8_t* vst, bool do_k, bool do_v) const {
    using C = Cfg<D>;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = threadIdx.x + i * NT;
      if (!EXACT && p >= C::TOT) continue;
      const int pv = p - C::KP;
      const bool isk = p < C::KP;
      if (isk ? !do_k : !do_v) continue;
      const int row = isk ? p / C::KPARTS : (pv >> 1);
      const int c0 = 2 * (isk ? p % C::KPARTS : (pv & 1));
      uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
      if (isk) {            // K codes -> fp8 e4m3 (QK runs on the fp8 MFMA)
        unpack_e4m3(r[i][0], h0, l0);
        unpack_e4m3(r[i][1], h1, l1);
        unpack_e4m3(r[i][2], h2, l2);
        unpack_e4m3(r[i][3], h3, l3);
      } else {              // V codes -> 16 * code int8 (PV runs on the i8 MFMA)
        unpack_x16(r[i][0], h0, l0);
        unpack_x16(r[i][1], h1, l1);
        unpack_x16(r[i][2], h2, l2);
        unpack_x16(r[i][3], h3, l3);
      }
      uint8_t* base = isk ? kst : vst;
      const int o0 = isk ? swz<D>(row, c0) : swz<64>(row, c0);
      const int o1 = isk ? swz<D>(row, c0 + 1) : swz<64>(row, c0 + 1);
      *reinterpret_cast<v4u*>(base + o0) = v4u{h0, h1, l0, l1};
      *reinterpret_cast<v4u*>(base + o1) = v4u{h2, h3, l2, l3};
    }
  }
};

// Q operands (B operand of S^T = K Q^T on the fp8 MFMA): query `q`,
// channels 64qc + 32hf + 0..31 as e4m3 bytes.
template <int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int bh, int q, int hf,
                                       v8i (&qop)[Cfg<D>::QC]) {
#pragma unroll
  for (int qc = 0; qc < Cfg<D>::QC; ++qc) {
    v4u w = v4u{0u, 0u, 0u, 0u};
    if (q < a.Npad)
      w = *reinterpret_cast<const v4u*>(a.qp + ((size_t)bh * a.Npad + q) * (D / 2) + (qc * 4 + hf * 2) * 8);
    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
    unpack_e4m3(w[0], h0, l0);
    unpack_e4m3(w[1], h1, l1);
    unpack_e4m3(w[2], h2, l2);
    unpack_e4m3(w[3], h3, l3);
    qop[qc] = v8i{(int)h0, (int)h1, (int)l0, (int)l1, (int)h2, (int)h3, (int)l2, (int)l3};
  }
}

// Key index (within the 64-key step) of accumulator register r of M-tile mt.
__device__ __forceinline__ int acc_key(int mt, int r, int hf) {
  return mt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
}

// ---- building blocks of one 64-key step for the 32 queries of a wave ------

// S^T of the step (exact integers in fp32): kst is the step's fp8 K tile.
template <int D>
__device__ __forceinline__ void qk_step(const uint8_t* kst, const v8i (&qop)[Cfg<D>::QC], v16f (&s)[2]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mt][r] = 0.0f;
#pragma unroll
    for (int qc = 0; qc < Cfg<D>::QC; ++qc) {
      const int row = mt * 32 + ln, c0 = qc * 4 + hf * 2;
      const v4i k0 = *reinterpret_cast<const v4i*>(kst + swz<D>(row, c0));
      const v4i k1 = *reinterpret_cast<const v4i*>(kst + swz<D>(row, c0 + 1));
      const v8i ka = v8i{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      s[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, qop[qc], s[mt], 0, 0, 0, 0, 0, 0);
    }
  }
}

// Keys at or past `nvalid` (ragged last step) are excluded from the max.
__device__ __forceinline__ void mask_scores(v16f (&s)[2], int nvalid) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (acc_key(mt, r, hf) >= nvalid) s[mt][r] = -INFINITY;
}

// Running-max candidate of the step for this lane's query (grid units):
// the smallest float >= max_j S_j * c.
__device__ __forceinline__ float step_max(const v16f (&s)[2], float c) {
  float mx = s[0][0];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
  mx = xhalf_max_f(mx);
  return mul_round_up(mx, c);
}

// P codes of M-tile mt (u = code + 8) as the 16-byte B operand of the PV MFMA.
__device__ __forceinline__ void pmap_mtile(const v16f& s, float c, float m, uint32_t (&p)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t acc = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float dlt = __builtin_fmaf(s[4 * i + e], c, -m);
      const float x = __builtin_rintf(dlt);
      acc = pmap_insert(x, (uint32_t)e, acc);
    }
    p[i] = acc;
  }
}

__device__ __forceinline__ void mask_codes(uint32_t (&p)[2][4], int nvalid) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (acc_key(mt, r, hf) >= nvalid) p[mt][r >> 2] &= ~(0xFFu << (8 * (r & 3)));
}

__device__ __forceinline__ uint32_t code_sum(const uint32_t (&p)[4], uint32_t U) {
#pragma unroll
  for (int i = 0; i < 4; ++i) U = __builtin_amdgcn_sad_u8(p[i], 0u, U);
  return U;
}

// O^T += V^T P^T for K-step ks (keys 32ks..32ks+31) of the step.
template <int D>
__device__ __forceinline__ void pv_kstep(const uint8_t* vst, const uint32_t (&p)[4], int ks,
                                         v16i (&acc)[Cfg<D>::DT]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  const v4i pb = v4i{(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::DT; ++dt) {
    const v4i va = *reinterpret_cast<const v4i*>(vst + swz<64>(dt * 32 + ln, ks * 2 + hf));
    acc[dt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(va, pb, acc[dt], 0, 0, 0);
  }
}

// The running max rises from st.m to m_new: fold the integer accumulator into
// the fp32 one with the rescale, A = (A + I) * beta, L = (L + U) * beta.
template <int D>
__device__ __forceinline__ void rescale(State<D>& st, float m_new) {
  const int lane = threadIdx.x & 63;
  const float beta = exp2f((st.m - m_new) * kInvPGrid);
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::DT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v4f* pa = reinterpret_cast<v4f*>(st.accf) + (dt * 4 + g) * 64 + lane;
      v4f acc = *pa;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = (acc[e] + (float)st.acc_i[dt][4 * g + e]) * beta;
        st.acc_i[dt][4 * g + e] = 0;
      }
      *pa = acc;
    }
  st.L = (st.L + (float)st.U) * beta;
  st.U = 0u;
}

// c = f32(f32(s_q s_k) alpha_G): grid units per unit of integer score.
__device__ __forceinline__ float score_scale(float cq, float sk, float alpha_g) {
  const float sqk = cq * sk;
  return sqk * alpha_g;
}

// One whole 64-key step in program order (used by the parity dump kernel;
// the main kernel runs the same blocks software-pipelined).
template <int D, bool DUMP>
__device__ __forceinline__ void tile_step(const uint8_t* kst, const uint8_t* vst,
                                          const v8i (&qop)[Cfg<D>::QC], float cq, float alpha_g,
                                          float sk, int nvalid, State<D>& st,
                                          const TileDumpArgs* dump, int wave) {
  using C = Cfg<D>;
  const int lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  v16f s[2];
  qk_step<D>(kst, qop, s);
  if (nvalid < kBlock) mask_scores(s, nvalid);
  const float cp = score_scale(cq, sk, alpha_g);
  const float m_new = fmaxf(st.m, step_max(s, cp));
  if (__ballot(m_new > st.m) != 0) rescale<D>(st, m_new);
  st.m = m_new;
  uint32_t p[2][4];
  pmap_mtile(s[0], cp, m_new, p[0]);
  pmap_mtile(s[1], cp, m_new, p[1]);
  if (nvalid < kBlock) mask_codes(p, nvalid);
  st.U = code_sum(p[0], st.U);
  st.U = code_sum(p[1], st.U);
  pv_kstep<D>(vst, p[0], 0, st.acc_i);
  pv_kstep<D>(vst, p[1], 1, st.acc_i);

  if (DUMP) {
    // Exact per-step integers: S, P codes, PV = sum (u - 8) vhat, running max.
    const int qrow = wave * 32 + ln;
    const v16i z = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    v16i pv[C::DT], cs[C::DT];
    uint32_t ones[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = acc_key(mt, r, hf);
        if (r % 4 == 0) ones[mt][r >> 2] = 0u;
        if (key < nvalid) ones[mt][r >> 2] |= 1u << (8 * (r & 3));
        const int sv = key < nvalid ? (int)s[mt][r] : 0;
        const int code = (int)((p[mt][r >> 2] >> (8 * (r & 3))) & 0xFFu) - 8;
        dump->s_int[qrow * 64 + key] = sv;
        dump->p_code[qrow * 64 + key] = (int8_t)code;
      }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) { pv[dt] = z; cs[dt] = z; }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pv_kstep<D>(vst, p[ks], ks, pv);
      pv_kstep<D>(vst, ones[ks], ks, cs);
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = dt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        dump->pv_int[qrow * D + d] = (pv[dt][r] - 8 * cs[dt][r]) / 16;
      }
    if (hf == 0) dump->m_after[qrow] = st.m;
  }
}

template <int D>
__device__ __forceinline__ void state_init(State<D>& st, float* accf) {
#pragma unroll
  for (int dt = 0; dt < Cfg<D>::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc_i[dt][r] = 0;
  st.m = -INFINITY;
  st.L = 0.0f;
  st.U = 0u;
  st.accf = accf;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < Cfg<D>::DT * 4; ++i)
    reinterpret_cast<v4f*>(accf)[i * 64 + lane] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(512) void k_int4_attn(AttnArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::KT + 2 * C::VT + 8 * C::ACCF];
  uint8_t* const kbuf = smem;                     // 2 K stages
  uint8_t* const vbuf = smem + 2 * C::KT;         // 2 V stages

  // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
  // contiguous range of (head, query-tile) ids.
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int full = nwg & ~7;
  const int lid = wg < full ? (wg & 7) * (full >> 3) + (wg >> 3) : wg;
  const int bh = lid / a.nqt, qt = lid % a.nqt;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  const int q0 = qt * 256 + wave * 32;
  const int qblk = q0 >> 6;
  const int nkb = a.nkb;

  v8i qop[C::QC];
  load_q<D>(a, bh, q0 + ln, hf, qop);
  const float cq = qblk < a.nblk ? a.s_q[(size_t)bh * a.nblk + qblk] : 0.0f;
  const float* sk = a.s_k + (size_t)bh * a.nblk;

  State<D> st;
  state_init<D>(st, reinterpret_cast<float*>(smem + 2 * C::KT + 2 * C::VT + wave * C::ACCF));

  // Pipeline: during step t the wave computes S of step t+1 (K one stage
  // ahead) while it turns S of step t into P codes, then P x V of step t;
  // one barrier per step.  K of step t+2 and V of step t+1 are fetched
  // during step t and widened into the stages freed by step t-1.
  TileLoad<D, 512> ld;
  ld.fetch(a, bh, 0, -1);
  ld.store(kbuf, vbuf, true, false);
  __syncthreads();
  ld.fetch(a, bh, nkb > 1 ? 1 : -1, 0);
  v16f s_cur[2];
  qk_step<D>(kbuf, qop, s_cur);
  const int nv0 = min(kBlock, a.N);
  if (nv0 < kBlock) mask_scores(s_cur, nv0);
  float cp_cur = score_scale(cq, sk[0], a.alpha_g);
  st.m = step_max(s_cur, cp_cur);
  ld.store(kbuf + C::KT, vbuf, nkb > 1, true);
  __syncthreads();

  // One pipelined step; the two score register sets swap roles every step
  // (the loop is unrolled by two so that no copy is needed).
  auto step = [&](v16f (&sc)[2], v16f (&sn)[2], int t) {
    ld.fetch(a, bh, t + 2 < nkb ? t + 2 : -1, t + 1 < nkb ? t + 1 : -1);
    const uint8_t* kst = kbuf + ((t + 1) & 1) * C::KT;
    const uint8_t* vst = vbuf + (t & 1) * C::VT;

    qk_step<D>(kst, qop, sn);                     // S of step t+1 (unused after the last step)
    uint32_t p[2][4];
    pmap_mtile(sc[0], cp_cur, st.m, p[0]);
    pmap_mtile(sc[1], cp_cur, st.m, p[1]);
    const int nvalid = min(kBlock, a.N - t * kBlock);
    if (nvalid < kBlock) mask_codes(p, nvalid);
    st.U = code_sum(p[0], st.U);
    st.U = code_sum(p[1], st.U);
    pv_kstep<D>(vst, p[0], 0, st.acc_i);
    pv_kstep<D>(vst, p[1], 1, st.acc_i);

    if (t + 1 < nkb) {
      const int nv1 = min(kBlock, a.N - (t + 1) * kBlock);
      if (nv1 < kBlock) mask_scores(sn, nv1);
      const float cp_next = score_scale(cq, sk[t + 1], a.alpha_g);
      const float m_new = fmaxf(st.m, step_max(sn, cp_next));
      if (__ballot(m_new > st.m) != 0) rescale<D>(st, m_new);
      st.m = m_new;
      cp_cur = cp_next;
    }
    ld.store(kbuf + (t & 1) * C::KT, vbuf + ((t + 1) & 1) * C::VT, t + 2 < nkb, t + 1 < nkb);
    __syncthreads();
  };
  v16f s_alt[2];
  int t = 0;
  for (; t + 1 < nkb; t += 2) {
    step(s_cur, s_alt, t);
    step(s_alt, s_cur, t + 1);
  }
  if (t < nkb) step(s_cur, s_alt, t);

  // o = A s_v / (16 L): the x16 of the widened V codes and the 1/15 of the
  // dequantized P cancel against the quantized row sum.
  const float lw = st.L + (float)st.U;
  const float lt = xhalf_sum_f(lw);
  const float inv = 1.0f / (16.0f * lt);
  const int q = q0 + ln;
  if (q < a.N) {
    const int b = bh / a.H, h = bh % a.H;
    const size_t obase = (((size_t)b * a.N + q) * a.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = dt * 32 + 8 * g + 4 * hf;
        const v4f sv = *reinterpret_cast<const v4f*>(a.s_v + (size_t)bh * D + d);
        const v4f af = reinterpret_cast<const v4f*>(st.accf)[(dt * 4 + g) * 64 + lane];
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = (af[e] + (float)st.acc_i[dt][4 * g + e]) * sv[e] * inv;
        if (OUT_BF16) {
          uint16_t* op = static_cast<uint16_t*>(a.out) + obase + d;
          *reinterpret_cast<uint2*>(op) =
              make_uint2((uint32_t)f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16),
                         (uint32_t)f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16));
        } else {
          float* op = static_cast<float*>(a.out) + obase + d;
          *reinterpret_cast<float4*>(op) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
  }
}

// Debug: the same per-step building blocks for the 64 queries of one Q
// block, in program order, dumping step kv_blk.  Two waves, one stage.
template <int D>
__global__ __launch_bounds__(128) void k_int4_tile_dump(AttnArgs a, TileDumpArgs t) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::KT + C::VT + 2 * C::ACCF];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hf = lane >> 5, ln = lane & 31;
  const int bh = t.bh;
  const int q0 = t.q_blk * kBlock + wave * 32;
  v8i qop[C::QC];
  load_q<D>(a, bh, q0 + ln, hf, qop);
  const float cq = a.s_q[(size_t)bh * a.nblk + t.q_blk];
  State<D> st;
  state_init<D>(st, reinterpret_cast<float*>(smem + C::KT + C::VT + wave * C::ACCF));
  TileLoad<D, 128> ld;
  for (int kb = 0; kb <= t.kv_blk; ++kb) {
    ld.fetch(a, bh, kb, kb);
    ld.store(smem, smem + C::KT, true, true);
    __syncthreads();
    const int nvalid = min(kBlock, a.N - kb * kBlock);
    const float sk = a.s_k[(size_t)bh * a.nblk + kb];
    if (kb == t.kv_blk)
      tile_step<D, true>(smem, smem + C::KT, qop, cq, a.alpha_g, sk, nvalid, st, &t, wave);
    else
      tile_step<D, false>(smem, smem + C::KT, qop, cq, a.alpha_g, sk, nvalid, st, nullptr, wave);
    __syncthreads();
  }
}

__global__ void k_pmap_probe(const float* __restrict__ x, uint8_t* __restrict__ u, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) u[i] = (uint8_t)(pmap_insert(x[i], 0u, 0u) & 0xFFu);
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

void launch_int4_attn(const AttnArgs& a, int D, bool out_bf16, int B, hipStream_t st) {
  const unsigned nwg = (unsigned)(B * a.H * a.nqt);
  if (D == 128) {
    if (out_bf16) k_int4_attn<128, true><<<nwg, 512, 0, st>>>(a);
    else k_int4_attn<128, false><<<nwg, 512, 0, st>>>(a);
  } else {
    if (out_bf16) k_int4_attn<64, true><<<nwg, 512, 0, st>>>(a);
    else k_int4_attn<64, false><<<nwg, 512, 0, st>>>(a);
  }
}

void launch_int4_tile_dump(const AttnArgs& a, const TileDumpArgs& t, int D, hipStream_t st) {
  if (D == 128) k_int4_tile_dump<128><<<1, 128, 0, st>>>(a, t);
  else k_int4_tile_dump<64><<<1, 128, 0, st>>>(a, t);
}

void launch_pmap_probe(const float* x, uint8_t* u, int64_t n, hipStream_t st) {
  if (n <= 0) return;
  k_pmap_probe<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(x, u, n);
}

void launch_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16) k_copy16<<<2048, 256, 0, st>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  const size_t rem = bytes - n16 * 16;
  if (rem) k_copy1<<<1, 256, 0, st>>>(static_cast<const uint8_t*>(src) + n16 * 16,
                                      static_cast<uint8_t*>(dst) + n16 * 16, rem);
}

}  // namespace ra
