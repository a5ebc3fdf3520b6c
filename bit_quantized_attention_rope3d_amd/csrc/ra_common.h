// ra_common.h -- device-side building blocks shared by the RotateAttention
// kernels for gfx950 (CDNA4).  Internal to libra_attn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));

constexpr int kBlock = 64;          // tokens per Q/K scale block and per key step
constexpr int kWave = 64;

// Code layout in the workspace, shared by the prologue (writer) and the
// attention kernels (readers).  gfx950 has no INT4 matrix instruction, so
// every INT4 code (Q, K, V in [-7, 7]) is stored already in the operand
// format of the f8f6f4 MFMA that consumes it, chosen once here rather than
// converted in each query tile of the attention: fp6 e2m3, which is exact
// for integers in [-7, 7].
//   * Q/K: fp6 e2m3 (6 bits per code), in tiles of 64 tokens (one scale
//     block).  A tile holds D/32 channel groups; the 32 codes of (token r,
//     group g) form 192 bits, code i at bits [6i, 6i+6), which is the
//     operand one lane supplies for a 64-deep contraction chunk.  Bits
//     0..127 of (r, g) are the 16 bytes at (64 g + r) * 16, bits 128..191
//     the 8 bytes at (D/32) * 1024 + (64 g + r) * 8: one 64-token tile is
//     48 * D bytes, read with one 16-byte and one 8-byte access per lane,
//     consecutive tokens at consecutive addresses.
//   * V: fp6 e2m3 tiles of one 64-key block (below, v6_*), the codes of
//     each channel in the slot order of the PV MFMA.
//   Slot s = 32*hf + 16*mt + j (j < 16) carries key 32*mt + 8*(j/4) + 4*hf +
//   (j%4): the key that the 32x32 accumulator of M-tile mt of S^T = K Q^T
//   leaves in register j of lane half hf.  Lane half hf supplies the bytes
//   of slots 32*hf..32*hf+31 of the PV MFMA's fp8 B operand, so the P codes
//   of a lane are that operand as they stand, with no shuffle.
__host__ __device__ constexpr int qk6_tile_bytes(int D) { return 48 * D; }
__host__ __device__ constexpr int qk6_lo_off(int r, int g) { return (64 * g + r) * 16; }
__host__ __device__ constexpr int qk6_hi_off(int D, int r, int g) { return (D / 32) * 1024 + (64 * g + r) * 8; }

// V tile of one 64-key block in fp6 e2m3, the A operand of the PV MFMA
// (whose B operand, the P codes, is fp8).  For channel d and lane half hf
// the 32 codes one lane supplies form 192 bits, code f at bits [6f, 6f+6):
// bits 0..127 at (D hf + d) * 16, bits 128..191 at 32 D + (D hf + d) * 8;
// 48 D bytes per tile, consecutive channels at consecutive addresses.  In
// this mixed fp6 x fp8 product, code f of lane half hf meets the P byte of
// slot 32 (f / 16) + 16 hf + f % 16 (lane layout of
// v_mfma_f32_32x32x64_f8f6f4 with an fp6 A and an fp8 B operand, measured
// with a probe: a lane half of the fp6 operand covers 16-slot pieces of
// both halves of the fp8 one).
__host__ __device__ constexpr int v6_tile_bytes(int D) { return 48 * D; }
__host__ __device__ constexpr int v6_lo_off(int D, int d, int hf) { return (D * hf + d) * 16; }
__host__ __device__ constexpr int v6_hi_off(int D, int d, int hf) { return 32 * D + (D * hf + d) * 8; }
__host__ __device__ constexpr int v6_slot(int hf, int f) { return 32 * (f >> 4) + 16 * hf + (f & 15); }

__host__ __device__ constexpr int slot_key_pv(int slot) {
  return 32 * ((slot >> 4) & 1) + 8 * ((slot & 15) >> 2) + 4 * (slot >> 5) + (slot & 3);
}

// bf16 path: 16-slot K-steps; slot s = 16*ks + 8*hf + j carries key
// 32*(ks/2) + 8*(2*(ks%2) + j/4) + 4*hf + (j%4).
__host__ __device__ constexpr int slot_key_bf16(int slot) {
  return 32 * (slot >> 5) + 8 * (2 * ((slot >> 4) & 1) + ((slot & 7) >> 2)) +
         4 * ((slot >> 3) & 1) + (slot & 3);
}

// OCP fp6 e2m3 code (bits 0..5) of an integer c in [-7, 7] (exact): sign in
// bit 5, |c| = 0..7 -> 00 08 10 14 18 1A 1C 1E.
__host__ __device__ constexpr uint32_t e2m3_of_code(int c) {
  return (c < 0 ? 0x20u : 0u) | (uint32_t)((0x1E1C1A1814100800ull >> (8 * (c < 0 ? -c : c))) & 0xFFu);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Combine the values of lanes l and l^32 (the two halves of a wave hold the
// same query columns).  v_permlane32_swap returns, per lane, its own value in
// one result and its partner's in the other, so a symmetric op of both
// results is the cross-half reduction whichever half the lane is in.
__device__ __forceinline__ float xhalf_max_f(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum_f(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Segment tables for 3D RoPE: cos/sin of segment s at [pos * (seg[s]/2) + pair].
struct RopeTabs {
  const float2* csn[3];   // per segment: (cos, sin) of pos * theta_j at [pos * pairs + j]
  int seg[3];
  int off[3];
  int dims[3];   // F, H, W
};

}  // namespace ra
