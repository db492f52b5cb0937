// Device-side helpers shared by the W12 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w12 {

typedef short short2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 256;  // 4 waves per workgroup for every kernel here

// Storage order of the planes: tiles of 16 rows x 128 columns, row-tile-major (rows padded with
// zero bytes to a multiple of 16).  Inside a tile, lane l = r + 16*g of a wave (row r, column
// group g = columns 32g..32g+31) owns:
//   AE bytes of columns 32g + 16h .. +16 at byte 1024*h + 16*l          (h = 0, 1)
//   B bytes of columns 32g .. +32 (16 bytes, four R1 groups of 8) at 16*l
//   dense bf16 (baseline) columns 32g + 8q .. +8 at byte 1024*q + 16*l   (q = 0..3)
// so each of these wave-wide 128-bit loads reads 1 KiB of contiguous memory, and the lane's
// data is exactly what the 16x16x32 MFMA operand layout wants for row r.
constexpr int kTileRows = 16;
constexpr int kTileCols = 128;
constexpr int kTileAE = 2048;   // bytes of AE per tile
constexpr int kTileLO = 1024;   // bytes of B per tile
constexpr int kTileBF = 4096;   // bytes of dense bf16 per tile

// Selectors for v_perm_b32 (bytes 0-3 come from the second source, 4-7 from the first,
// 0x0C yields a zero byte).  Each builds a pair of 16-bit halves, one per weight, whose high
// byte is the weight's AE byte and whose low byte carries its B nibble in bits 7..4.
constexpr uint32_t kSelPair01 = 0x05010400u;  // AE bytes 0,1 over source bytes 0,1
constexpr uint32_t kSelPair23 = 0x07030602u;  // AE bytes 2,3 over source bytes 2,3
constexpr uint32_t kSelQ01 = 0x050C040Cu;     // AE bytes 0,1, zero low bytes (B := 0)
constexpr uint32_t kSelQ23 = 0x070C060Cu;     // AE bytes 2,3, zero low bytes

// An opaque copy of 0x38003800 held in a VGPR.  With the AND mask in an SGPR this lets the
// compiler fold mask-and-insert into one v_and_or_b32 (gfx9 VOP3 takes no literals and one
// scalar operand).
__device__ __forceinline__ uint32_t exp112_pair() {
  uint32_t v = 0x38003800u;
  asm volatile("" : "+v"(v));
  return v;
}

// Two weights of one row -> two bfloat16 "window" values w' in one dword.
// Input half (per weight): AE byte in bits 15..8 = s | E(4) | m6..4, B nibble in bits 7..4.
// An arithmetic shift by 4 gives s s s s s | E | m6..4 | B; clearing bit 14 and setting bits
// 13..11 turns the five sign copies into s 0 1 1 1, i.e. exponent field 0111 EEEE = 112 + E.
// So w' = (-1)^s * 2^(E - 15) * (1 + m/128): the weight divided by 2^(base - 112).
__device__ __forceinline__ uint32_t window_pair(uint32_t ae_word, uint32_t lo_word, uint32_t sel,
                                                uint32_t exp112) {
  uint32_t u = __builtin_amdgcn_perm(ae_word, lo_word, sel);
  short2v s = __builtin_bit_cast(short2v, u) >> (short2v){4, 4};
  return (__builtin_bit_cast(uint32_t, s) & 0xBFFFBFFFu) | exp112;
}

// Eight consecutive weights (AE words a0: k0..3, a1: k4..7; B word lo for the group) ->
// four dwords of w' pairs (k0,k1) (k2,k3) (k4,k5) (k6,k7).  The B word holds nibble i of the
// group at bit 8*(i%4) + 4*(i/4), so the low nibbles (weights 0..3) need one shift by 4 and
// the high nibbles (weights 4..7) none.
__device__ __forceinline__ void window_group8(uint32_t a0, uint32_t a1, uint32_t lo, uint32_t exp112,
                                              uint32_t out[4]) {
  const uint32_t lo4 = lo << 4;
  out[0] = window_pair(a0, lo4, kSelPair01, exp112);
  out[1] = window_pair(a0, lo4, kSelPair23, exp112);
  out[2] = window_pair(a1, lo, kSelPair01, exp112);
  out[3] = window_pair(a1, lo, kSelPair23, exp112);
}

// The 8-bit view alone (Q pass): same as window_group8 with every B nibble 0.
__device__ __forceinline__ void window_group8_q(uint32_t a0, uint32_t a1, uint32_t exp112,
                                                uint32_t out[4]) {
  out[0] = window_pair(a0, a0, kSelQ01, exp112);
  out[1] = window_pair(a0, a0, kSelQ23, exp112);
  out[2] = window_pair(a1, a1, kSelQ01, exp112);
  out[3] = window_pair(a1, a1, kSelQ23, exp112);
}

// 2^(base - 112) as a float: the factor from w' back to the true weight.  base is 1..239,
// so the exponent field base + 15 is 16..254 (always a normal float).
__device__ __forceinline__ float window_scale(uint32_t base) {
  return __uint_as_float((base + 15u) << 23);
}

// w' of an escaped slot (AE = 0, B = 0): exponent 112, mantissa 0 -> 2^-15.
constexpr float kPlaceholder = 3.0517578125e-05f;
// The same slot in the midpoint Q pass (format 3 of the launch interface: B read as 8):
// 2^-15 * (1 + 8/128).
constexpr float kPlaceholderMid = 3.24249267578125e-05f;
template <int FMT>
constexpr float placeholder_of() { return FMT == 3 ? kPlaceholderMid : kPlaceholder; }
// Whether an escaped slot contributes a placeholder that the escape patch must take back out:
// every format but the 8-bit copy (format 4), whose escaped slots hold the code 0.
template <int FMT>
constexpr bool has_placeholder() { return FMT != 4; }

// Sixteen signed 8-bit codes (one 128-bit word, columns in order) -> eight dwords of bfloat16
// pairs (c0, c1) (c2, c3) ...: each code converts exactly to float (a sign-extended byte select),
// and a code of magnitude <= 127 has at most 7 significant bits, so the float's high half is the
// exact bfloat16; one byte permute packs two of them.
__device__ __forceinline__ void i8_group16(u32x4 v, uint32_t out[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wd = v[i];
    const float f0 = (float)(int8_t)(wd & 0xFFu);
    const float f1 = (float)(int8_t)((wd >> 8) & 0xFFu);
    const float f2 = (float)(int8_t)((wd >> 16) & 0xFFu);
    const float f3 = (float)(int8_t)(wd >> 24);
    out[2 * i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    out[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  }
}

// Midpoint Q pass: the B nibble of both bfloat16 halves of each decoded pair set to 8.
__device__ __forceinline__ void midpoint16(uint32_t p[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] |= 0x00080008u;
}

// float -> bfloat16 bits, round to nearest, ties to even (NaN stays NaN, quieted)
__device__ __forceinline__ uint16_t float_to_bf16_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// silu(z) = z / (1 + e^-z) in float (e^-z overflowing to +Inf gives the limit -0)
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// Non-temporal 128-bit load: weight planes are streamed once, keep them out of the caches'
// reuse set.
template <typename T>
__device__ __forceinline__ T load_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

// ---- buffer loads (raw buffer resources) ----
// An offset at or past a buffer's num_records reads zeros and fetches nothing, so a kernel can
// issue every load of a software pipeline unconditionally (no load behind a branch, static ring
// registers) and switch a load off by its offset alone.
constexpr uint32_t kOOB = 0x80000000u;      // offset past every range used here
constexpr int kAuxNT = 2;                   // cache policy bits: non-temporal (weights stream once)

typedef __amdgpu_buffer_rsrc_t Rsrc;

// Raw buffer over `bytes` bytes at `p` (stride 0, 32-bit data format word of the gfx9 family).
__device__ __forceinline__ Rsrc make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Forces the 16 decoded words to exist here: a decode is pure arithmetic, which the optimizer
// would otherwise sink to its first use -- past the refill of the ring slot it reads, which then
// needs other registers and a copy back (after a wait) at the end of every loop body.
__device__ __forceinline__ void pin16(uint32_t p[16]) {
  asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]),
               "+v"(p[6]), "+v"(p[7]), "+v"(p[8]), "+v"(p[9]), "+v"(p[10]), "+v"(p[11]),
               "+v"(p[12]), "+v"(p[13]), "+v"(p[14]), "+v"(p[15]));
}

// Workgroup barrier that orders LDS only (vector-memory loads in flight are not waited for).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace w12
