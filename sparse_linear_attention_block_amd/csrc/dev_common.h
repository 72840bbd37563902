// Device helpers shared by the gfx950 kernels: bf16 <-> f32, MFMA wrappers,
// wave reductions. Wave size is 64 on CDNA4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));
typedef int i32x8 __attribute__((__vector_size__(8 * sizeof(int))));

__device__ __forceinline__ float bf2f(uint32_t u16) { return __uint_as_float(u16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 with round-to-nearest-even (the native gfx950 conversion)
__device__ __forceinline__ uint32_t f2bf(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// D += A * B with A: 16x32, B: 32x16 bf16, D: 16x16 f32.
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and
// D[4*(l/16) + r][l%16] in register r. Any permutation of the 32 k slots is
// allowed as long as A and B use the same one.
__device__ __forceinline__ f32x4 mfma_bf16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D += A * B with A: 16x64, B: 64x16 int8, D: 16x16 int32; lane l holds 16
// consecutive k of row/column l%16 at k offset 16*(l/16).
__device__ __forceinline__ i32x4 mfma_i8(const uint4& a, const uint4& b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// D += A * B with A: 16x128, B: 128x16 fp8 e4m3 (OCP), D: 16x16 f32; lane l
// holds 32 k of row/column l%16 (unit block scales).
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// The same with a per-lane E8M0 block scale on B: the 32 k values lane l holds
// of column l%16 are multiplied by 2^(sb - 127) (A keeps unit scales).
__device__ __forceinline__ f32x4 mfma_fp8_sb(const i32x8& a, const i32x8& b, f32x4 c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

__device__ __forceinline__ float wave_max16(float v) {  // over the 16 lanes of a row group
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}
// over lanes l, l^16, l^32, l^48 (the four k groups of one MFMA column)
__device__ __forceinline__ float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float group4_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Feature map elu(x) + 1 (elementwise): x + 1 above zero, exp(x) at or below
// (the hardware base-2 exponential of x log2(e)).
__device__ __forceinline__ float elu1(float x) {
  return x > 0.f ? x + 1.0f : __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

}  // namespace sla

namespace sla {

typedef short s16x4_t __attribute__((__vector_size__(4 * sizeof(short))));

// D += A * B with A: 16x16, B: 16x16 bf16, D: 16x16 f32. Lane l holds
// A[l%16][4*(l/16) .. +3], B[4*(l/16) .. +3][l%16], D as in mfma_bf16.
__device__ __forceinline__ f32x4 mfma_bf16_k16(const uint2& a, const uint2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (other counters left alone), gfx9 encoding.
constexpr int waitcnt_vm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// 16-byte asynchronous copy global -> LDS: lane l writes lds_wave_base + 16*l.
__device__ __forceinline__ void load_lds16(const void* gptr, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gptr, (void __attribute__((address_space(3)))*)lds_wave_base,
                                   16, 0, 0);
}

// Raw buffer resource over `bytes` bytes from `base` (stride 0, 32-bit data
// format word of the gfx9 descriptor). Copies through it take a per-lane 32-bit
// offset and a wave-uniform scalar offset, so moving to the next tile costs no
// vector instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16-byte asynchronous copy of base + soff + voff into LDS: lane l writes lds_wave_base + 16*l.
__device__ __forceinline__ void load_lds16_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff,
                                               void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (void __attribute__((address_space(3)))*)lds_wave_base, 16, (int)voff, soff, 0, 0);
}

}  // namespace sla

namespace sla {

// s_waitcnt immediate that waits for this wave's LDS (and scalar memory)
// operations only; vector-memory operations may stay in flight.
constexpr int kWaitLgkm0 = 0xf | (0x3 << 14) | (0x7 << 4) | (0x0 << 8);

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes are
// complete, then all waves meet. Unlike __syncthreads() it does not wait for
// outstanding global loads (such as asynchronous global->LDS copies of the next
// tile), which must be waited for explicitly before their data is read.
__device__ __forceinline__ void lds_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

}  // namespace sla

namespace sla {

// float -> OCP fp8 e4m3 (finite, max 448) with round-to-nearest-even and
// saturation: the hardware conversion rounds to nearest even but turns
// magnitudes above 464 into NaN, so the input is clamped to +-448 first.
// Returns the byte in the low 8 bits.
__device__ __forceinline__ uint32_t f2e4m3(float x) {
  x = fminf(fmaxf(x, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xffu;
}
// four floats -> four e4m3 bytes in one word (element 0 in the low byte)
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  c = fminf(fmaxf(c, -448.0f), 448.0f);
  d = fminf(fmaxf(d, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// four floats known to lie in [-448, 448] (up to rounding, below the 464 at
// which the conversion would give NaN) -> four e4m3 bytes, no clamp
__device__ __forceinline__ uint32_t pack_e4m3x4_nosat(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// symmetric int8 code: round-to-nearest-even of x * inv, clamped to +-127
__device__ __forceinline__ int q_i8(float x, float inv) {
  return (int)fminf(fmaxf(__builtin_rintf(x * inv), -127.0f), 127.0f);
}

}  // namespace sla

namespace sla {

// Workgroup L of T (dispatched round-robin over the 8 XCDs) -> logical index:
// each XCD gets a contiguous range of logical indices, so neighbouring tiles
// share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int L, int T) {
  const int q = T >> 3, rm = T & 7;
  const int x = L & 7, pos = L >> 3;
  return x * q + min(x, rm) + pos;
}

// Compacts the indices j with mrow[j] == value, ascending, into list; returns the count.
__device__ inline int compact_row(const int8_t* __restrict__ mrow, int Nb, int8_t value,
                           uint16_t* list, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int total = 0;
  for (int base = 0; base < Nb; base += 256) {
    const int j = base + tid;
    const bool f = (j < Nb) && (mrow[j] == value);
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (f) list[off + before] = (uint16_t)j;
    total += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  return total;
}

typedef short s16x4_v __attribute__((ext_vector_type(4)));

// Row-major tiles of d-wide bf16 rows (K, V, H_i^T, Q, dO rows) sit in LDS
// with their 16-byte chunks XOR-swizzled by the row: chunk c of row r at
// position c ^ row_swz(r). At d = 128 (16 chunks, one row spans all 64 banks)
// row_swz(r) = 2 ((r % 8) ^ 4 h) + h with h = (r / 8) % 2, found by measuring
// LDS bank conflicts of both reads the kernels make on gfx950:
//  - a transposed read (ds_read_b64_tr_b16) takes 32-byte chunk pairs from
//    8 consecutive rows per 256-byte cycle, so those rows must sit on 8
//    distinct pairs: the pair index row_swz(r) / 2 = (r % 8) ^ 4 h is a
//    permutation of r % 8 for either h;
//  - a 16-byte fragment read (ds_read_b128) of 16 rows at one chunk is free
//    of conflicts only when rows r and r + 8 fall in different 128-byte
//    halves of the row (the 4 h term).
// The plain r % 16 swizzle meets the second and costs the first two extra
// cycles per read; (r % 8) << 1 | h the reverse. At d = 64 it is r % 8.
template <int D>
__device__ __forceinline__ int row_swz(int r) {
  if constexpr (D == 128) {
    const int h = (r >> 3) & 1;
    return (((r & 7) ^ (h << 2)) << 1) | h;
  } else {
    return r & (D / 8 - 1);
  }
}

// The A operand of O^T += V^T P^T for feature tile ft of a 32-key step (or any
// product that contracts over 32 rows held row-major in LDS), from the step's V
// rows in LDS (row-major; 16-byte chunk q of row r at position
// q ^ row_swz(r), like the K rows): lane (l16, g) holds feature 16 ft + l16 of keys
// 4g .. 4g+3 (k slots 0-3) and 16+4g .. 16+4g+3 (k slots 4-7), the key order of
// P^T's B operand. gfx950's transposed LDS read gives lane i of a 16-lane group
// element k of source lane 4k + i/4's four 16-bit values at position i % 4, so
// source lane s reads the 8 bytes of features 16 ft + 4 (s % 4) .. +3 of key
// row 4g + s / 4 (and of the row 16 below it). xb is the lane's byte offset for
// ft = 0; the swizzle and the row occupy disjoint bits, so tile ft is at
// xb ^ 32 ft.
template <int D>
__device__ __forceinline__ int vt_base(int g, int s) {
  const int r = 4 * g + (s >> 2), m = row_swz<D>(r);
  return r * 2 * D + 32 * (m >> 1) + 16 * (((s & 3) >> 1) ^ (m & 1)) + 8 * (s & 1);
}
template <int D>
__device__ __forceinline__ uint4 vt_frag(const uint16_t* vrows, int xb, int ft) {
  const char* p0 = reinterpret_cast<const char*>(vrows) + (xb ^ (32 * ft));
  const char* p1 = p0 + 16 * 2 * D;  // 16 key rows further
  const s16x4_v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_v*)p0);
  const s16x4_v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_v*)p1);
  const uint2 lo = __builtin_bit_cast(uint2, a), hi = __builtin_bit_cast(uint2, b);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// The same compaction in two parts, so that a kernel can load the mask row
// first, issue its other prologue loads, and wait only for the mask: mask_load
// reads bytes j = tid + NT k of the row for k < kMaskPre (every load is issued;
// indices past the row re-read its last byte and are ignored), compact_loaded
// builds the list from them with one barrier for all chunks; rows longer than
// NT kMaskPre blocks finish chunk by chunk as in compact_row. NT is the
// workgroup's thread count (a multiple of 64); wsum holds (NT / 64) kMaskPre ints.
constexpr int kMaskPre = 8;
template <int NT = 256>
__device__ __forceinline__ void mask_load(const int8_t* __restrict__ mrow, int Nb,
                                          int8_t (&mv)[kMaskPre]) {
#pragma unroll
  for (int k = 0; k < kMaskPre; ++k) mv[k] = mrow[min((int)threadIdx.x + NT * k, Nb - 1)];
}
template <int NT = 256>
__device__ inline int compact_loaded(const int8_t (&mv)[kMaskPre], const int8_t* __restrict__ mrow,
                                     int Nb, int8_t value, uint16_t* list, int* wsum) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int before[kMaskPre];
  uint32_t fbits = 0;
#pragma unroll
  for (int k = 0; k < kMaskPre; ++k) {
    const bool f = tid + NT * k < Nb && mv[k] == value;
    const uint64_t bal = __ballot(f);
    before[k] = __popcll(bal & ((1ull << lane) - 1ull));
    fbits |= (uint32_t)f << k;
    if (lane == 0) wsum[NW * k + wave] = __popcll(bal);
  }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int k = 0; k < kMaskPre; ++k) {
    int off = total;
    for (int w = 0; w < wave; ++w) off += wsum[NW * k + w];
    if ((fbits >> k) & 1) list[off + before[k]] = (uint16_t)(tid + NT * k);
#pragma unroll
    for (int w = 0; w < NW; ++w) total += wsum[NW * k + w];
  }
  __syncthreads();
  for (int base = NT * kMaskPre; base < Nb; base += NT) {
    const int j = base + tid;
    const bool f = (j < Nb) && (mrow[j] == value);
    const uint64_t bal = __ballot(f);
    const int bef = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (f) list[off + bef] = (uint16_t)j;
#pragma unroll
    for (int w = 0; w < NW; ++w) total += wsum[w];
    __syncthreads();
  }
  return total;
}

}  // namespace sla
