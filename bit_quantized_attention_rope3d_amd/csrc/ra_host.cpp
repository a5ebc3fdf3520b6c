// ra_host.cpp -- host runtime behind include/ra_attn.h: validation, plans,
// RoPE tables, workspace layout, launches, error reporting, the step/block
// schedule and the parity exports.
//
// Method source: "RotateAttention: RoPE-Aware Rotation and Range Rectification
// for INT4 Quantized Attention in Video Generation" (pith.science review):
// Sec. 3 / Fig. 2 (3D RoPE segments), Sec. 4.1 / Fig. 3 (Interleaved rotation
// merged into RoPE), Sec. 4.2 (P map), Sec. 5.1 (FP16 step/block fallback).
#include "ra_attn.h"

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "ra_kernels.h"

namespace {

thread_local std::string g_err;

ra_status fail(ra_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

ra_status ok() {
  g_err.clear();
  return RA_OK;
}

// RA_FAULT_INJECT=alloc|launch forces the matching failure path (host-side
// tests of error mapping).
bool inject(const char* what) {
  const char* e = std::getenv("RA_FAULT_INJECT");
  return e && std::strcmp(e, what) == 0;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- P map thresholds ([RA] Sec. 4.2: u = round(P p), p = 2^d, half up) --
//
// In terms of x = -d >= 0, u = #{k : x <= X_k} where X_k is the largest
// binary32 x with P 2^-x >= k + 1/2.  Non-negative binary32 values are
// ordered like their bit patterns, so X_k is found by bisection over bit
// patterns between 0 (P 2^0 = P >= k + 1/2 for k < P) and 8 (P 2^-8 < 1/2),
// the condition evaluated with a 64-bit-significand exp2l.
float pmap_boundary(int P, int k) {
  uint32_t lo = 0u, hi = 0x41000000u;   // bits of 0.0f and 8.0f
  auto holds = [&](uint32_t b) {
    float x;
    std::memcpy(&x, &b, 4);
    return (long double)P * exp2l(-(long double)x) >= (long double)k + 0.5L;
  };
  while (hi - lo > 1u) {
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (holds(mid)) lo = mid;
    else hi = mid;
  }
  float x;
  std::memcpy(&x, &lo, 4);
  return x;
}

// The attention kernels' table cell of x: rint(4096 x), ties to even (the
// rounding the kernels' subnormal multiply performs; 4096 x is exact in
// binary64).
int pmap_cell(float x) { return (int)std::nearbyint((double)x * 4096.0); }

ra::PMapArgs pmap_args(int p_mode) {
  ra::PMapArgs pm{};
  pm.P = p_mode ? 7 : 15;
  for (int k = 0; k < pm.P; ++k) {
    const float xk = pmap_boundary(pm.P, k);
    pm.cell[k] = pmap_cell(xk);
    pm.ythr[k] = xk * 0.125f;
    if (pmap_cell(std::nextafter(xk, INFINITY)) == pm.cell[k]) pm.split |= 1u << k;
  }
  // The first even cell past X_0's: every x from there on has u = 0.  Even,
  // so that rint(top - 4096 x), the kernels' reversed address, is exactly
  // top - rint(4096 x) at ties as well.
  pm.top = (pm.cell[0] + 2) & ~1;
  pm.top_sub = std::ldexp((float)pm.top, -149);
  return pm;
}

// e4m3 byte of an integer 0 <= u <= 15 (exact): the PV operand format of u.
uint8_t e4m3_of_uint(uint32_t u) {
  if (u == 0 || u > 15) return 0;
  int e = 0;
  while ((u >> (e + 1)) != 0) ++e;                       // floor(log2 u) <= 3
  return (uint8_t)(((e + 7) << 3) | ((u << (3 - e)) & 7u));
}

// The kernels' P-map table (layout in ra_kernels.h, kPTabTotal bytes): the
// entry at address a is for cell j = top - a; it counts the X_k whose cell
// lies above j, plus the X_k whose cell is j when that cell holds nothing
// above X_k; a cell that does is marked 0x80 | k.  Addresses past top stay 0.
std::vector<uint8_t> pmap_table(const ra::PMapArgs& pm) {
  std::vector<uint8_t> t(ra::kPTabTotal, 0);
  for (int a = 0; a <= pm.top; ++a) {
    const int j = pm.top - a;
    uint32_t u = 0, mark = 0;
    for (int k = 0; k < pm.P; ++k) {
      const bool split = (pm.split >> k) & 1u;
      if (j < pm.cell[k] || (j == pm.cell[k] && !split)) ++u;
      if (j == pm.cell[k] && split) mark = 0x80u | (uint32_t)k;
    }
    t[a] = (uint8_t)(mark ? mark : e4m3_of_uint(u));
  }
  for (int k = 0; k < pm.P; ++k) {      // records k >= P stay zero
    std::memcpy(&t[ra::kPTabBytes + 8 * k], &pm.ythr[k], 4);
    t[ra::kPTabBytes + 8 * k + 4] = e4m3_of_uint((uint32_t)k);
    t[ra::kPTabBytes + 8 * k + 5] = e4m3_of_uint((uint32_t)k + 1);
  }
  return t;
}

// Bytes of RoPE tables in a plan's device buffer, rounded up to 16: the
// P-map table follows them.
size_t ptab_offset(size_t tab_floats) { return (tab_floats * sizeof(float) + 15) & ~(size_t)15; }

struct Layout {
  int N, Npad, nblk, nkb, nqt;
  size_t off_q, off_k, off_v, off_sq, off_sk, off_sv, off_vamax, off_dbg, total;
};

constexpr size_t kDbgBytes(int D) { return 64 * 64 * 4 + 64 * 64 + (size_t)64 * D * 4 + 64 * 4 + 1024; }

ra_status validate(const ra_shape* s, const ra_opts* o) {
  if (!s || !o) return fail(RA_ERR_INVALID_ARG, "shape and opts must be non-null");
  if (s->batch < 1 || s->heads < 1 || s->grid_f < 1 || s->grid_h < 1 || s->grid_w < 1)
    return fail(RA_ERR_SHAPE, "batch, heads and grid dims must be >= 1 (got B=%d H=%d grid=%dx%dx%d)",
                s->batch, s->heads, s->grid_f, s->grid_h, s->grid_w);
  const long long N = (long long)s->grid_f * s->grid_h * s->grid_w;
  if (N > (1LL << 26))
    return fail(RA_ERR_SHAPE, "token count %lld exceeds the supported 2^26", N);
  if ((long long)s->batch * s->heads * ((N + 255) / 256) > 0x7FFFFFFFLL)
    return fail(RA_ERR_SHAPE, "batch * heads * ceil(N/256) does not fit a launch grid");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", s->head_dim);
  for (int i = 0; i < 3; ++i)
    if (s->seg[i] < 2 || (s->seg[i] & 1))
      return fail(RA_ERR_SEGMENTS, "segment %d has length %d; RoPE segments must be even and >= 2",
                  i, s->seg[i]);
  if (s->seg[0] + s->seg[1] + s->seg[2] != s->head_dim)
    return fail(RA_ERR_SEGMENTS, "segments %d+%d+%d do not sum to head_dim %d", s->seg[0], s->seg[1],
                s->seg[2], s->head_dim);
  if (o->rot < RA_ROT_NONE || o->rot > RA_ROT_FULL)
    return fail(RA_ERR_INVALID_ARG, "rot %d is not a ra_rot", o->rot);
  if (o->prec != RA_PREC_INT4 && o->prec != RA_PREC_BF16)
    return fail(RA_ERR_INVALID_ARG, "prec %d is not a ra_prec", o->prec);
  if ((o->in_dtype != RA_DT_F32 && o->in_dtype != RA_DT_BF16) ||
      (o->out_dtype != RA_DT_F32 && o->out_dtype != RA_DT_BF16))
    return fail(RA_ERR_DTYPE, "dtypes must be RA_DT_F32 or RA_DT_BF16 (in=%d out=%d)", o->in_dtype,
                o->out_dtype);
  if (!(o->rope_theta > 0.0) || !std::isfinite(o->rope_theta))
    return fail(RA_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (!(o->softmax_scale >= 0.0) || !std::isfinite(o->softmax_scale))
    return fail(RA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (o->p_mode != 0 && o->p_mode != 1)
    return fail(RA_ERR_INVALID_ARG, "p_mode %d is not 0 (range-optimized) or 1 (symmetric)", o->p_mode);
  if (o->v_hadamard != 0 && o->v_hadamard != 1)
    return fail(RA_ERR_INVALID_ARG, "v_hadamard %d is not 0 or 1", o->v_hadamard);
  return RA_OK;
}

Layout layout_of(const ra_shape* s, const ra_opts* o) {
  Layout L{};
  L.N = s->grid_f * s->grid_h * s->grid_w;
  L.nblk = (L.N + ra::kBlock - 1) / ra::kBlock;
  L.nkb = L.nblk;
  L.Npad = L.nblk * ra::kBlock;
  L.nqt = (L.N + 255) / 256;
  const size_t BH = (size_t)s->batch * s->heads, D = s->head_dim;
  const size_t A = 256;
  size_t off = 0;
  if (o->prec == RA_PREC_INT4) {
    const size_t qk = BH * L.nblk * (size_t)ra::qk6_tile_bytes((int)D);   // fp6 tiles
    const size_t vb = BH * L.nkb * (size_t)ra::v6_tile_bytes((int)D);     // fp6 tiles
    L.off_q = off; off = align_up(off + qk, A);
    L.off_k = off; off = align_up(off + qk, A);
    L.off_v = off; off = align_up(off + vb, A);
    L.off_sq = off; off = align_up(off + BH * L.nblk * 4, A);
    L.off_sk = off; off = align_up(off + BH * L.nblk * 4, A);
    L.off_sv = off; off = align_up(off + BH * D * 4, A);
    L.off_vamax = off; off = align_up(off + BH * D * 4, A);
    L.off_dbg = off; off = align_up(off + kDbgBytes((int)D), A);
  } else {
    const size_t tens = BH * L.Npad * D * 2;
    L.off_q = off; off = align_up(off + tens, A);
    L.off_k = off; off = align_up(off + tens, A);
    L.off_v = off; off = align_up(off + tens, A);
    L.off_sq = L.off_sk = L.off_sv = L.off_vamax = L.off_dbg = off;
  }
  L.total = off;
  return L;
}

}  // namespace

struct ra_plan_s {
  ra_shape shape;
  ra_opts opts;
  Layout lay;
  int off[3];
  std::vector<float> cs[3], sn[3];
  size_t tab_floats;
  float alpha;
  ra::PMapArgs pm;
  std::mutex mu;
  std::map<int, float*> dev_tabs;
};

namespace {

// cos/sin of pos * theta^(-2j/L) (+ pi/4 when the Interleaved rotation is
// merged), angles in binary64, each value rounded once to binary32.
void build_tables(ra_plan_s* p) {
  const int dims[3] = {p->shape.grid_f, p->shape.grid_h, p->shape.grid_w};
  const bool merged = p->opts.prec == RA_PREC_INT4 && p->opts.rot == RA_ROT_INTERLEAVED;
  p->tab_floats = 0;
  int off = 0;
  for (int s = 0; s < 3; ++s) {
    const int L = p->shape.seg[s], half = L / 2;
    p->off[s] = off;
    off += L;
    p->cs[s].resize((size_t)dims[s] * half);
    p->sn[s].resize((size_t)dims[s] * half);
    for (int pos = 0; pos < dims[s]; ++pos)
      for (int j = 0; j < half; ++j) {
        const double e = (double)(-2 * j) / (double)L;
        const double freq = std::pow(p->opts.rope_theta, e);
        double ang = (double)pos * freq;
        if (merged) {
          const double quarter = M_PI / 4.0;
          ang = ang + quarter;
        }
        p->cs[s][(size_t)pos * half + j] = (float)std::cos(ang);
        p->sn[s][(size_t)pos * half + j] = (float)std::sin(ang);
      }
    p->tab_floats += 2 * p->cs[s].size();
  }
}

// Copy the plan's RoPE tables to the current device, once per device
// (allocates and synchronises: called from ra_plan_create and
// ra_plan_upload, never from the forward entry points).
ra_status upload_tables(ra_plan p) {
  if (inject("alloc")) return fail(RA_ERR_OOM, "injected allocation failure (RA_FAULT_INJECT=alloc)");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(RA_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> g(p->mu);
  if (p->dev_tabs.count(dev)) return RA_OK;
  float* buf = nullptr;
  const size_t bytes = ptab_offset(p->tab_floats) + ra::kPTabTotal;
  if (hipMalloc(&buf, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(RA_ERR_OOM, "hipMalloc of %zu bytes of plan tables failed", bytes);
  }
  // (cos, sin) interleaved, one 8-byte load per pair, then the P-map table.
  std::vector<uint8_t> host(bytes, 0);
  size_t o = 0;
  for (int s = 0; s < 3; ++s)
    for (size_t i = 0; i < p->cs[s].size(); ++i) {
      std::memcpy(&host[o], &p->cs[s][i], 4);
      std::memcpy(&host[o + 4], &p->sn[s][i], 4);
      o += 8;
    }
  const std::vector<uint8_t> pt = pmap_table(p->pm);
  std::memcpy(&host[ptab_offset(p->tab_floats)], pt.data(), pt.size());
  if (hipMemcpy(buf, host.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    hipFree(buf);
    return fail(RA_ERR_HIP, "copying plan tables to device %d failed", dev);
  }
  p->dev_tabs[dev] = buf;
  return RA_OK;
}

// The current device's copy of the P-map table (no allocation, no copy).
ra_status device_ptab(ra_plan p, const uint8_t** t) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(RA_ERR_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> g(p->mu);
  auto it = p->dev_tabs.find(dev);
  if (it == p->dev_tabs.end())
    return fail(RA_ERR_INVALID_ARG,
                "the plan has no tables on device %d: create it with that device current, "
                "or call ra_plan_upload there first", dev);
  *t = reinterpret_cast<const uint8_t*>(it->second) + ptab_offset(p->tab_floats);
  return RA_OK;
}

// The current device's copy of the tables (no allocation, no copy).
ra_status device_tables(ra_plan p, ra::RopeTabs* t) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(RA_ERR_HIP, "hipGetDevice failed");
  float* buf = nullptr;
  {
    std::lock_guard<std::mutex> g(p->mu);
    auto it = p->dev_tabs.find(dev);
    if (it == p->dev_tabs.end())
      return fail(RA_ERR_INVALID_ARG,
                  "the plan has no tables on device %d: create it with that device current, "
                  "or call ra_plan_upload there first", dev);
    buf = it->second;
  }
  const int dims[3] = {p->shape.grid_f, p->shape.grid_h, p->shape.grid_w};
  size_t o = 0;
  for (int s = 0; s < 3; ++s) {
    t->csn[s] = reinterpret_cast<const float2*>(buf + o);
    o += 2 * p->cs[s].size();
    t->seg[s] = p->shape.seg[s];
    t->off[s] = p->off[s];
    t->dims[s] = dims[s];
  }
  return RA_OK;
}

bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

ra_status check_ws(ra_plan p, void* ws, size_t ws_bytes) {
  if (!ws) return fail(RA_ERR_WORKSPACE, "workspace is null");
  if (misaligned(ws)) return fail(RA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  if (ws_bytes < p->lay.total)
    return fail(RA_ERR_WORKSPACE, "workspace has %zu bytes; this plan needs %zu", ws_bytes, p->lay.total);
  return RA_OK;
}

ra_status after_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return RA_OK;
}

ra::AttnArgs attn_args(ra_plan p, uint8_t* ws, void* o) {
  ra::AttnArgs a{};
  a.qp = ws + p->lay.off_q;
  a.kp = ws + p->lay.off_k;
  a.vp = ws + p->lay.off_v;
  a.s_q = reinterpret_cast<const float*>(ws + p->lay.off_sq);
  a.s_k = reinterpret_cast<const float*>(ws + p->lay.off_sk);
  a.s_v = reinterpret_cast<const float*>(ws + p->lay.off_sv);
  a.out = o;
  a.N = p->lay.N;
  a.H = p->shape.heads;
  a.Npad = p->lay.Npad;
  a.nblk = p->lay.nblk;
  a.nkb = p->lay.nkb;
  a.nqt = p->lay.nqt;
  a.alpha = p->alpha;
  a.p_mode = p->opts.p_mode;
  a.v_hadamard = p->opts.v_hadamard;
  a.pm = p->pm;
  a.row_dbg = nullptr;
  return a;
}

}  // namespace

extern "C" {

ra_status ra_opts_default(ra_opts* o) {
  if (!o) return fail(RA_ERR_INVALID_ARG, "opts is null");
  std::memset(o, 0, sizeof *o);
  o->rot = RA_ROT_HALF;
  o->prec = RA_PREC_INT4;
  o->in_dtype = RA_DT_BF16;
  o->out_dtype = RA_DT_F32;
  o->rope_theta = 10000.0;
  o->softmax_scale = 0.0;
  o->p_mode = 0;
  o->v_hadamard = 0;
  return ok();
}

ra_status ra_plan_create(const ra_shape* shape, const ra_opts* opts, ra_plan* out) {
  if (!out) return fail(RA_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  ra_status st = validate(shape, opts);
  if (st != RA_OK) return st;
  ra_plan p = new (std::nothrow) ra_plan_s();
  if (!p) return fail(RA_ERR_OOM, "host allocation of the plan failed");
  p->shape = *shape;
  p->opts = *opts;
  p->lay = layout_of(shape, opts);
  const double scale = opts->softmax_scale > 0.0 ? opts->softmax_scale : 1.0 / std::sqrt((double)shape->head_dim);
  p->alpha = (float)(M_LOG2E * scale);
  p->pm = pmap_args(opts->p_mode);
  if (p->pm.top + 1 > ra::kPTabEntries) {
    delete p;
    return fail(RA_ERR_UNSUPPORTED, "P-map table needs %d entries (built for %d)", p->pm.top + 1,
                ra::kPTabEntries);
  }
  build_tables(p);
  // Tables go to the current device now, so that the forward calls neither
  // allocate nor synchronise.  With no device present the plan still serves
  // the host-side queries.
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) {
    (void)hipGetLastError();
    ndev = 0;
  }
  if (ndev > 0) {
    st = upload_tables(p);
    if (st != RA_OK) {
      delete p;
      return st;
    }
    void* ws = nullptr;   // resolve the no-allocation workspace of this device now
    if (ra::noalloc_scratch(&ws) != hipSuccess) (void)hipGetLastError();
  }
  *out = p;
  return ok();
}

ra_status ra_plan_upload(ra_plan p) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "plan is null");
  ra_status st = upload_tables(p);
  return st == RA_OK ? ok() : st;
}

ra_status ra_plan_destroy(ra_plan p) {
  if (!p) return ok();
  for (auto& kv : p->dev_tabs) {
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess && hipSetDevice(kv.first) == hipSuccess) {
      hipFree(kv.second);
      hipSetDevice(cur);
    }
  }
  delete p;
  return ok();
}

ra_status ra_plan_workspace_size(ra_plan p, size_t* bytes) {
  if (!p || !bytes) return fail(RA_ERR_INVALID_ARG, "plan and bytes must be non-null");
  *bytes = p->lay.total;
  return ok();
}

ra_status ra_workspace_size(const ra_shape* shape, const ra_opts* opts, size_t* bytes) {
  if (!bytes) return fail(RA_ERR_INVALID_ARG, "bytes is null");
  ra_status st = validate(shape, opts);
  if (st != RA_OK) return st;
  *bytes = layout_of(shape, opts).total;
  return ok();
}

ra_status ra_attn_prologue(ra_plan p, const void* q, const void* k, const void* v, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "plan is null");
  if (!q || !k || !v) return fail(RA_ERR_INVALID_ARG, "q, k and v must be non-null");
  if (misaligned(q) || misaligned(k) || misaligned(v))
    return fail(RA_ERR_ALIGNMENT, "q, k and v must be 16-byte aligned");
  ra_status st = check_ws(p, ws, ws_bytes);
  if (st != RA_OK) return st;
  if (inject("launch")) return fail(RA_ERR_HIP, "injected launch failure (RA_FAULT_INJECT=launch)");
  ra::RopeTabs tabs;
  st = device_tables(p, &tabs);
  if (st != RA_OK) return st;

  uint8_t* w = static_cast<uint8_t*>(ws);
  const int D = p->shape.head_dim;
  const bool in_bf16 = p->opts.in_dtype == RA_DT_BF16;
  ra::QKPrologueArgs qa{};
  qa.q = q;
  qa.k = k;
  qa.q_out = w + p->lay.off_q;
  qa.k_out = w + p->lay.off_k;
  qa.s_q = reinterpret_cast<float*>(w + p->lay.off_sq);
  qa.s_k = reinterpret_cast<float*>(w + p->lay.off_sk);
  qa.tabs = tabs;
  qa.B = p->shape.batch;
  qa.N = p->lay.N;
  qa.H = p->shape.heads;
  qa.Npad = p->lay.Npad;
  qa.nblk = p->lay.nblk;
  ra::VQuantArgs vq{};
  vq.v = v;
  vq.vamax = reinterpret_cast<const uint32_t*>(w + p->lay.off_vamax);
  vq.v_out = w + p->lay.off_v;
  vq.s_v = reinterpret_cast<float*>(w + p->lay.off_sv);
  vq.N = p->lay.N;
  vq.H = p->shape.heads;
  vq.nkb = p->lay.nkb;
  if (p->opts.prec == RA_PREC_INT4) {
    ra::VAmaxArgs va{};
    va.v = v;
    va.vamax = reinterpret_cast<uint32_t*>(w + p->lay.off_vamax);
    va.N = p->lay.N;
    va.H = p->shape.heads;
    va.chunk = 512;
    ra::launch_int4_prologue(qa, va, vq, D, p->opts.rot, in_bf16, p->opts.v_hadamard != 0, stream);
  } else {
    ra::launch_bf16_prologue(qa, vq, D, in_bf16, stream);
  }
  st = after_launch("prologue");
  return st == RA_OK ? ok() : st;
}

ra_status ra_attn_main(ra_plan p, void* o, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "plan is null");
  if (!o) return fail(RA_ERR_INVALID_ARG, "o must be non-null");
  if (misaligned(o)) return fail(RA_ERR_ALIGNMENT, "o must be 16-byte aligned");
  ra_status st = check_ws(p, ws, ws_bytes);
  if (st != RA_OK) return st;
  if (inject("launch")) return fail(RA_ERR_HIP, "injected launch failure (RA_FAULT_INJECT=launch)");
  ra::AttnArgs a = attn_args(p, static_cast<uint8_t*>(ws), o);
  if (p->opts.prec == RA_PREC_INT4 && (st = device_ptab(p, &a.ptab)) != RA_OK) return st;
  const bool out_bf16 = p->opts.out_dtype == RA_DT_BF16;
  if (p->opts.prec == RA_PREC_INT4)
    ra::launch_int4_attn(a, p->shape.head_dim, out_bf16, p->shape.batch, stream);
  else
    ra::launch_bf16_attn(a, p->shape.head_dim, out_bf16, p->shape.batch, stream);
  st = after_launch("attention");
  return st == RA_OK ? ok() : st;
}

ra_status ra_attn_fwd(ra_plan p, const void* q, const void* k, const void* v, void* o, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  if (!o) return fail(RA_ERR_INVALID_ARG, "o must be non-null");
  if (misaligned(o)) return fail(RA_ERR_ALIGNMENT, "o must be 16-byte aligned");
  ra_status st = ra_attn_prologue(p, q, k, v, ws, ws_bytes, stream);
  if (st != RA_OK) return st;
  return ra_attn_main(p, o, ws, ws_bytes, stream);
}

ra_status ra_attn_fwd_noalloc(ra_plan p, const void* q, const void* k, const void* v, void* o,
                              hipStream_t stream) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "plan is null");
  if (p->lay.total > (size_t)RA_NOALLOC_WORKSPACE_BYTES)
    return fail(RA_ERR_WORKSPACE,
                "this plan needs a %zu-byte workspace; the no-allocation entry point holds at most %zu "
                "bytes (use ra_attn_fwd with a caller workspace)",
                p->lay.total, (size_t)RA_NOALLOC_WORKSPACE_BYTES);
  void* ws = nullptr;
  const hipError_t e = ra::noalloc_scratch(&ws);
  if (e != hipSuccess)
    return fail(RA_ERR_HIP, "looking up the device workspace failed: %s", hipGetErrorString(e));
  return ra_attn_fwd(p, q, k, v, o, ws, (size_t)RA_NOALLOC_WORKSPACE_BYTES, stream);
}

ra_status ra_attn_fwd_simple(const void* q, const void* k, const void* v, void* o, int32_t batch,
                             int32_t heads, int32_t head_dim, int32_t grid_f, int32_t grid_h,
                             int32_t grid_w, int32_t seg_f, int32_t seg_h, int32_t seg_w, int32_t rot,
                             int32_t prec, int32_t in_dtype, int32_t out_dtype, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  static std::mutex mu;
  static std::map<std::vector<int32_t>, ra_plan> cache;
  ra_shape s{batch, heads, head_dim, grid_f, grid_h, grid_w, {seg_f, seg_h, seg_w}};
  ra_opts op;
  ra_opts_default(&op);
  op.rot = rot;
  op.prec = prec;
  op.in_dtype = in_dtype;
  op.out_dtype = out_dtype;
  ra_status st = validate(&s, &op);
  if (st != RA_OK) return st;
  std::vector<int32_t> key{batch, heads, head_dim, grid_f, grid_h, grid_w, seg_f, seg_h, seg_w,
                           rot, prec, in_dtype, out_dtype};
  ra_plan p = nullptr;
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      p = it->second;
    } else {
      st = ra_plan_create(&s, &op, &p);
      if (st != RA_OK) return st;
      cache[key] = p;
    }
  }
  return ra_attn_fwd(p, q, k, v, o, ws, ws_bytes, stream);
}

ra_prec ra_schedule_pick(const ra_schedule* s, int32_t step, int32_t n_steps, int32_t block,
                         int32_t n_blocks) {
  if (!s) return RA_PREC_BF16;
  const bool step_full = step < s->steps_head || step >= n_steps - s->steps_tail;
  const bool block_full = block < s->blocks_head || block >= n_blocks - s->blocks_tail;
  return (step_full || block_full) ? RA_PREC_BF16 : RA_PREC_INT4;
}

const char* ra_status_str(ra_status s) {
  switch (s) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID_ARG: return "RA_ERR_INVALID_ARG";
    case RA_ERR_SHAPE: return "RA_ERR_SHAPE";
    case RA_ERR_SEGMENTS: return "RA_ERR_SEGMENTS";
    case RA_ERR_DTYPE: return "RA_ERR_DTYPE";
    case RA_ERR_ALIGNMENT: return "RA_ERR_ALIGNMENT";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_OOM: return "RA_ERR_OOM";
    case RA_ERR_HIP: return "RA_ERR_HIP";
  }
  return "RA_ERR_UNKNOWN";
}

const char* ra_last_error_message(void) { return g_err.c_str(); }

ra_status ra_pmap_thresholds(int32_t p_mode, float* T) {
  if (p_mode != 0 && p_mode != 1) return fail(RA_ERR_INVALID_ARG, "p_mode %d is not 0 or 1", p_mode);
  if (!T) return fail(RA_ERR_INVALID_ARG, "T is null");
  const ra::PMapArgs pm = pmap_args(p_mode);
  for (int k = 0; k < pm.P; ++k) T[k] = -pmap_boundary(pm.P, k);
  return ok();
}

static_assert(RA_PMAP_TABLE_BYTES == ra::kPTabTotal, "exported P-map table size");

ra_status ra_pmap_table(int32_t p_mode, uint8_t* out, size_t bytes, int32_t* top) {
  if (p_mode != 0 && p_mode != 1) return fail(RA_ERR_INVALID_ARG, "p_mode %d is not 0 or 1", p_mode);
  if (!out || !top) return fail(RA_ERR_INVALID_ARG, "out and top must be non-null");
  if (bytes < (size_t)ra::kPTabTotal)
    return fail(RA_ERR_INVALID_ARG, "buffer of %zu bytes is shorter than the %d-byte table", bytes, ra::kPTabTotal);
  const ra::PMapArgs pm = pmap_args(p_mode);
  const std::vector<uint8_t> t = pmap_table(pm);
  std::memcpy(out, t.data(), t.size());
  *top = pm.top;
  return ok();
}

ra_status ra_debug_prologue(ra_plan p, const void* q, const void* k, const void* v, void* ws,
                            size_t ws_bytes, int8_t* q_codes, float* s_q, int8_t* k_codes,
                            float* s_k, int8_t* v_codes, float* s_v, hipStream_t stream) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "plan is null");
  if (p->opts.prec != RA_PREC_INT4) return fail(RA_ERR_UNSUPPORTED, "debug prologue needs an INT4 plan");
  if (!q_codes || !s_q || !k_codes || !s_k || !v_codes || !s_v)
    return fail(RA_ERR_INVALID_ARG, "host output buffers must be non-null");
  ra_status st = ra_attn_prologue(p, q, k, v, ws, ws_bytes, stream);
  if (st != RA_OK) return st;
  if (hipStreamSynchronize(stream) != hipSuccess) return fail(RA_ERR_HIP, "prologue failed on device");
  const Layout& L = p->lay;
  const size_t BH = (size_t)p->shape.batch * p->shape.heads;
  const int D = p->shape.head_dim, N = L.N;
  const size_t qkb = BH * L.nblk * (size_t)ra::qk6_tile_bytes(D), tens = BH * L.nkb * (size_t)ra::v6_tile_bytes(D);
  std::vector<uint8_t> pq(qkb), pk(qkb), pv(tens);
  const uint8_t* w = static_cast<const uint8_t*>(ws);
  if (hipMemcpy(pq.data(), w + L.off_q, qkb, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(pk.data(), w + L.off_k, qkb, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(pv.data(), w + L.off_v, tens, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(s_q, w + L.off_sq, BH * L.nblk * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(s_k, w + L.off_sk, BH * L.nblk * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(s_v, w + L.off_sv, BH * D * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(RA_ERR_HIP, "copy of prologue outputs failed");
  // Encoded code -> integer code; encodings of no code in [-7, 7] decode to
  // -128, which no valid code equals.
  int8_t code_of6[64];
  for (int i = 0; i < 64; ++i) code_of6[i] = INT8_MIN;
  for (int c = -7; c <= 7; ++c) code_of6[ra::e2m3_of_code(c)] = (int8_t)c;
  // Code i of a 192-bit fp6 string (16 bytes, then 8).
  auto fp6_code = [&](const uint8_t* lo, const uint8_t* hi, int i) {
    uint8_t bits[24];
    std::memcpy(bits, lo, 16);
    std::memcpy(bits + 16, hi, 8);
    const int b0 = 6 * i;
    const unsigned v = (unsigned)bits[b0 / 8] | ((unsigned)(b0 / 8 + 1 < 24 ? bits[b0 / 8 + 1] : 0) << 8);
    return code_of6[(v >> (b0 % 8)) & 0x3Fu];
  };
  // Q/K: fp6 tiles of 64 tokens; (token r, group g) is 192 bits, code i at
  // bits [6i, 6i+6): 16 bytes at the lo offset, then 8 at the hi offset.
  const int tb = ra::qk6_tile_bytes(D);
  for (size_t bh = 0; bh < BH; ++bh)
    for (int n = 0; n < N; ++n) {
      const size_t tile = (bh * L.nblk + n / 64) * (size_t)tb;
      const int r = n % 64;
      for (int g = 0; g < D / 32; ++g)
        for (int which = 0; which < 2; ++which) {
          const uint8_t* t = (which ? pk.data() : pq.data()) + tile;
          int8_t* o = (which ? k_codes : q_codes) + (bh * N + n) * D + 32 * g;
          for (int i = 0; i < 32; ++i) o[i] = fp6_code(t + ra::qk6_lo_off(r, g), t + ra::qk6_hi_off(D, r, g), i);
        }
    }
  // V: per 64-key block, channel and lane half, 32 codes whose slots follow
  // the fp6 x fp8 lane layout of the PV MFMA.
  for (size_t bh = 0; bh < BH; ++bh)
    for (int kb = 0; kb < L.nkb; ++kb) {
      const uint8_t* t = pv.data() + (bh * L.nkb + kb) * (size_t)ra::v6_tile_bytes(D);
      for (int d = 0; d < D; ++d)
        for (int hf = 0; hf < 2; ++hf)
          for (int f = 0; f < 32; ++f) {
            const int key = kb * 64 + ra::slot_key_pv(ra::v6_slot(hf, f));
            if (key < N)
              v_codes[(bh * N + key) * D + d] = fp6_code(t + ra::v6_lo_off(D, d, hf), t + ra::v6_hi_off(D, d, hf), f);
          }
    }
  return ok();
}

ra_status ra_debug_tile(ra_plan p, void* ws, size_t ws_bytes, int32_t b, int32_t h, int32_t q_blk,
                        int32_t kv_blk, int32_t* s_int, int8_t* p_codes, int32_t* pv_int,
                        float* m_after, hipStream_t stream) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "plan is null");
  if (p->opts.prec != RA_PREC_INT4) return fail(RA_ERR_UNSUPPORTED, "debug tile needs an INT4 plan");
  if (!s_int || !p_codes || !pv_int || !m_after)
    return fail(RA_ERR_INVALID_ARG, "host output buffers must be non-null");
  if (b < 0 || b >= p->shape.batch || h < 0 || h >= p->shape.heads || q_blk < 0 ||
      q_blk >= p->lay.nblk || kv_blk < 0 || kv_blk >= p->lay.nkb)
    return fail(RA_ERR_INVALID_ARG, "tile index out of range");
  ra_status st = check_ws(p, ws, ws_bytes);
  if (st != RA_OK) return st;
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int D = p->shape.head_dim;
  ra::AttnArgs a = attn_args(p, w, nullptr);
  if ((st = device_ptab(p, &a.ptab)) != RA_OK) return st;
  ra::TileDumpArgs t{};
  uint8_t* dbg = w + p->lay.off_dbg;
  t.s_int = reinterpret_cast<int32_t*>(dbg);
  t.p_code = reinterpret_cast<int8_t*>(dbg + 64 * 64 * 4);
  t.pv_int = reinterpret_cast<int32_t*>(dbg + 64 * 64 * 5);
  t.m_after = reinterpret_cast<float*>(dbg + 64 * 64 * 5 + (size_t)64 * D * 4);
  t.bh = b * p->shape.heads + h;
  t.q_blk = q_blk;
  t.kv_blk = kv_blk;
  ra::launch_int4_tile_dump(a, t, D, stream);
  st = after_launch("tile dump");
  if (st != RA_OK) return st;
  if (hipStreamSynchronize(stream) != hipSuccess) return fail(RA_ERR_HIP, "tile dump failed on device");
  if (hipMemcpy(s_int, t.s_int, 64 * 64 * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(p_codes, t.p_code, 64 * 64, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(pv_int, t.pv_int, (size_t)64 * D * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(m_after, t.m_after, 64 * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(RA_ERR_HIP, "copy of tile dump failed");
  return ok();
}

ra_status ra_debug_row_digests(ra_plan p, void* o, void* ws, size_t ws_bytes, uint32_t* rows,
                               hipStream_t stream) {
  if (!p) return fail(RA_ERR_INVALID_ARG, "plan is null");
  if (p->opts.prec != RA_PREC_INT4) return fail(RA_ERR_UNSUPPORTED, "row digests need an INT4 plan");
  if (p->opts.out_dtype != RA_DT_F32) return fail(RA_ERR_UNSUPPORTED, "row digests need an f32-output plan");
  if (!o || !rows) return fail(RA_ERR_INVALID_ARG, "o and rows must be non-null");
  if (misaligned(o) || misaligned(rows)) return fail(RA_ERR_ALIGNMENT, "o and rows must be 16-byte aligned");
  ra_status st = check_ws(p, ws, ws_bytes);
  if (st != RA_OK) return st;
  ra::AttnArgs a = attn_args(p, static_cast<uint8_t*>(ws), o);
  if ((st = device_ptab(p, &a.ptab)) != RA_OK) return st;
  a.row_dbg = rows;
  ra::launch_int4_attn_rowdbg(a, p->shape.head_dim, p->shape.batch, stream);
  st = after_launch("attention (row digests)");
  return st == RA_OK ? ok() : st;
}

ra_status ra_debug_pmap(const float* d, uint8_t* u, int64_t n, int32_t p_mode, hipStream_t stream) {
  if (n < 0) return fail(RA_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && (!d || !u)) return fail(RA_ERR_INVALID_ARG, "d and u must be non-null");
  if (p_mode != 0 && p_mode != 1) return fail(RA_ERR_INVALID_ARG, "p_mode %d is not 0 or 1", p_mode);
  // The table the attention kernels use, built and copied to the current
  // device once per P mode (kept until the process ends).
  static std::mutex mu;
  static std::map<std::pair<int, int>, uint8_t*> tabs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(RA_ERR_HIP, "hipGetDevice failed");
  const ra::PMapArgs pm = pmap_args(p_mode);
  uint8_t* tab = nullptr;
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = tabs.find({dev, p_mode});
    if (it == tabs.end()) {
      const std::vector<uint8_t> h = pmap_table(pm);
      if (hipMalloc(&tab, h.size()) != hipSuccess) {
        (void)hipGetLastError();
        return fail(RA_ERR_OOM, "hipMalloc of the P-map table failed");
      }
      if (hipMemcpy(tab, h.data(), h.size(), hipMemcpyHostToDevice) != hipSuccess) {
        hipFree(tab);
        return fail(RA_ERR_HIP, "copying the P-map table failed");
      }
      tabs[{dev, p_mode}] = tab;
    } else {
      tab = it->second;
    }
  }
  ra::launch_pmap_probe(d, u, n, pm, tab, stream);
  ra_status st = after_launch("pmap probe");
  return st == RA_OK ? ok() : st;
}

ra_status ra_debug_tables(ra_plan p, int32_t seg, float* cos_out, float* sin_out) {
  if (!p || !cos_out || !sin_out) return fail(RA_ERR_INVALID_ARG, "null argument");
  if (seg < 0 || seg > 2) return fail(RA_ERR_INVALID_ARG, "seg must be 0, 1 or 2");
  std::memcpy(cos_out, p->cs[seg].data(), p->cs[seg].size() * sizeof(float));
  std::memcpy(sin_out, p->sn[seg].data(), p->sn[seg].size() * sizeof(float));
  return ok();
}

ra_status ra_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes && (!dst || !src)) return fail(RA_ERR_INVALID_ARG, "dst and src must be non-null");
  if (misaligned(dst) || misaligned(src)) return fail(RA_ERR_ALIGNMENT, "dst and src must be 16-byte aligned");
  ra::launch_copy(dst, src, bytes, stream);
  ra_status st = after_launch("copy");
  return st == RA_OK ? ok() : st;
}

ra_status ra_bench_mfma_peak(int32_t kind, int32_t iters, int32_t blocks, float* sink, uint64_t* clk,
                             double* ops_out, hipStream_t stream) {
  const int per = ra::mfma_peak_ops_per_instr(kind);
  if (per == 0) return fail(RA_ERR_INVALID_ARG, "unknown MFMA kind %d", kind);
  if (iters < 1 || blocks < 1) return fail(RA_ERR_INVALID_ARG, "iters and blocks must be >= 1");
  if (!sink || !clk || !ops_out) return fail(RA_ERR_INVALID_ARG, "null argument");
  *ops_out = (double)per * ra::mfma_peak_chains() * iters * 4.0 * blocks;
  ra::launch_mfma_peak(kind, iters, blocks, sink, clk, stream);
  ra_status st = after_launch("mfma peak");
  return st == RA_OK ? ok() : st;
}

}  // extern "C"
