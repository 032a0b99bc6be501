// Device-side building blocks shared by the GEMM kernels (w4_gemm.hip,
// w4_gemm_stream.hip): operand expansion of prepacked blocks, MFMA steps,
// epilogue helpers, bounded buffer loads, the XCD-aware tile order and the
// LDS-ring barrier.
#pragma once

#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

template <int OP>
struct OpTraits;
template <>
struct OpTraits<OP_I8> {
  using Acc = i32x4;
  static constexpr int kElemBytes = 1;
};
template <>
struct OpTraits<OP_FP8> {
  using Acc = f32x4;
  static constexpr int kElemBytes = 1;
};
template <>
struct OpTraits<OP_F16> {
  using Acc = f32x4;
  static constexpr int kElemBytes = 2;
};
template <>
struct OpTraits<OP_BF16> {
  using Acc = f32x4;
  static constexpr int kElemBytes = 2;
};

// 16-byte words of one lane's activation fragment for one 128-deep block.
template <int OP>
constexpr int act_vecs() {
  return OpTraits<OP>::kElemBytes * 2;  // 32 bytes (8-bit) or 64 bytes (16-bit)
}

// Expand one lane's four packed words into MFMA operand words.
template <int OP, bool FLIP>
__device__ __forceinline__ void expand_weights(const u32x4 w, const f16x2 nz, uint32_t e[16]) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (OP == OP_I8) {
      expand_i8x16(FLIP ? (q[j] ^ 0x88888888u) : q[j], e[2 * j], e[2 * j + 1]);
    } else if constexpr (OP == OP_FP8) {
      expand_fp8(FLIP ? (q[j] ^ 0x88888888u) : q[j], e[2 * j], e[2 * j + 1]);
    } else {
      expand_f16class<OP>(q[j], &e[4 * j]);
      if constexpr (OP == OP_F16) {
#pragma unroll
        for (int t = 0; t < 4; ++t) e[4 * j + t] = f16x2_add(e[4 * j + t], nz);
      }
    }
  }
}

template <int OP>
__device__ __forceinline__ void block_mma(const uint32_t e[16], const u32x4* a,
                                          typename OpTraits<OP>::Acc& acc) {
  if constexpr (OP == OP_I8) {
    acc = mma_i8(u32x4{e[0], e[1], e[2], e[3]}, a[0], acc);
    acc = mma_i8(u32x4{e[4], e[5], e[6], e[7]}, a[1], acc);
  } else if constexpr (OP == OP_FP8) {
    acc = mma_fp8(u32x8{e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]},
                  u32x8{a[0].x, a[0].y, a[0].z, a[0].w, a[1].x, a[1].y, a[1].z, a[1].w}, acc);
  } else {
#pragma unroll
    for (int kw = 0; kw < 4; ++kw) {
      const u32x4 wv{e[4 * kw], e[4 * kw + 1], e[4 * kw + 2], e[4 * kw + 3]};
      if constexpr (OP == OP_F16)
        acc = mma_f16(wv, a[kw], acc);
      else
        acc = mma_bf16(wv, a[kw], acc);
    }
  }
}

// bf16 W4A16: the operand holds 128 + c, so each group also needs the sum of
// its activations (times 128 + z).  A weight operand of ones gives that sum in
// every D row.
__device__ __forceinline__ void ones_mma(const u32x4* a, f32x4& ones) {
  const u32x4 one{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
  for (int kw = 0; kw < 4; ++kw) ones = mma_bf16(one, a[kw], ones);
}

// Asymmetric int8 W4A8: the operand holds 16 (u - 8) (the uint4b8
// expansion of the raw code u), so each group also needs 16 * sum(a), times
// z - 8, to reach 16 * sum(a (u - z)) exactly.  A weight operand of 16s gives
// that sum in every D row.
__device__ __forceinline__ void ones_mma_i8(const u32x4* a, i32x4& ones) {
  const u32x4 sixteen{0x10101010u, 0x10101010u, 0x10101010u, 0x10101010u};
  ones = mma_i8(sixteen, a[0], ones);
  ones = mma_i8(sixteen, a[1], ones);
}

// Groups smaller than a 128-deep block (W4A16, group size 64 or 32: SG = 2 or
// 4 sub-groups per block).  Lane group kq of an MFMA operand holds the k in
// [32 kq, 32 kq + 32) of the block, so the lanes of sub-group sg are those
// with kq / (4 / SG) == sg; an operand with the other lanes zeroed gives that
// sub-group's dot product.
template <int SG>
__device__ __forceinline__ int lane_subgroup(int kq) { return kq / (4 / SG); }

template <int N>
__device__ __forceinline__ void mask_words(const uint32_t* e, bool keep, uint32_t* out) {
#pragma unroll
  for (int t = 0; t < N; ++t) out[t] = keep ? e[t] : 0u;
}

// W4A16 with pre-scaled zero-points: the operand holds the raw code (fp16:
// 1024 + c - 1024; bf16: 128 + c), and each group subtracts zs * sum(a),
// the activation sum again from a ones-operand.
template <int OP>
__device__ __forceinline__ void ones_mma_16(const u32x4* a, f32x4& ones) {
  if constexpr (OP == OP_BF16) {
    ones_mma(a, ones);
  } else {
    const u32x4 one{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
    for (int kw = 0; kw < 4; ++kw) ones = mma_f16(one, a[kw], ones);
  }
}

// bf16 ones-operand restricted to the lanes that keep it: the activation sum
// of one sub-group.
__device__ __forceinline__ void ones_mma_masked(const u32x4* a, bool keep, f32x4& ones) {
  const uint32_t v = keep ? 0x3F803F80u : 0u;
  const u32x4 one{v, v, v, v};
#pragma unroll
  for (int kw = 0; kw < 4; ++kw) ones = mma_bf16(one, a[kw], ones);
}

// The group (or whole-K) dot product of one D element.
template <int OP>
__device__ __forceinline__ float partial_value(typename OpTraits<OP>::Acc acc, f32x4 ones, float zc,
                                               int i) {
  if constexpr (OP == OP_I8) return (float)acc[i] * 0.0625f;  // acc = 16 * sum
  if constexpr (OP == OP_BF16) return fmaf(-zc, ones[i], acc[i]);
  return acc[i];
}

// Integer group partial of the int8 path (acc holds 16 * sum); 0 otherwise.
template <int OP>
__device__ __forceinline__ int32_t int_partial(typename OpTraits<OP>::Acc acc, int i) {
  if constexpr (OP == OP_I8) return acc[i] >> 4;
  return 0;
}

__device__ __forceinline__ float zero_point(const GemmArgs& p, int64_t n, int g) {
  return p.z ? load_as_f32(p.z, p.z_dtype, n * p.G + g) : 8.0f;
}

__device__ __forceinline__ void store_out(const GemmArgs& p, int64_t m, int64_t n, float v) {
  if (p.out_dtype == W4_F16)
    static_cast<uint16_t*>(p.out)[m * p.N + n] = f32_to_f16_bits(v);
  else
    static_cast<uint16_t*>(p.out)[m * p.N + n] = f32_to_bf16_bits(v);
}

// Final epilogue of one element: v is the group-scaled total (grouped) or the
// raw whole-K dot product (per channel; int32 for the int8 path).
template <int OP, bool GROUPED>
__device__ __forceinline__ float finalize(const GemmArgs& p, int64_t m, int64_t n, float fv,
                                          int32_t iv) {
  float v;
  if constexpr (GROUPED) {
    v = fv;
  } else {
    const float s = load_as_f32(p.s, p.s_dtype, n);
    v = (OP == OP_I8) ? (float)iv * (s * 0.0625f) : fv * s;
  }
  if (p.a_scales) v *= p.a_scales[m];
  if (p.bias) v += load_as_f32(p.bias, p.out_dtype, n);
  return v;
}

__device__ __forceinline__ bool in_window(const GemmArgs& p, int64_t m, int64_t n) {
  return m >= p.m0 && m < p.m1 && n >= p.n0 && n < p.n1;
}

template <int OP>
__device__ __forceinline__ void store_partial(const GemmArgs& p, int g, int64_t m, int64_t n, float fv,
                                              int32_t iv) {
  const int64_t wm = p.m1 - p.m0, wn = p.n1 - p.n0;
  const int64_t idx = ((int64_t)g * wm + (m - p.m0)) * wn + (n - p.n0);
  if constexpr (OP == OP_I8)
    static_cast<int32_t*>(p.partials)[idx] = iv;
  else
    static_cast<float*>(p.partials)[idx] = fv;
}

// Buffer loads: a descriptor bounds every load, and an out-of-range offset
// returns zero without touching memory.
constexpr uint32_t kBufferDword3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)
constexpr uint32_t kOutOfRange = 0x80000000u;    // offset beyond every descriptor's size

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0LL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufferDword3);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Scale and zero-point loads without branches (a branch around a load makes
// the compiler wait for every outstanding load where the paths join): the
// 32-bit word holding element i is always loaded; the 16-bit half and the
// conversion are chosen by selects when the value is used.
__device__ __forceinline__ uint32_t elem_byte(int dtype, uint32_t i) { return dtype == W4_F32 ? i * 4u : i * 2u; }
__device__ __forceinline__ uint32_t load_word(__amdgpu_buffer_rsrc_t r, int dtype, uint32_t i, bool in) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)(in ? (elem_byte(dtype, i) & ~3u) : kOutOfRange), 0, 0);
}
__device__ __forceinline__ float word_to_f32(uint32_t w, int dtype, uint32_t i) {
  const uint32_t h = (elem_byte(dtype, i) & 2u) ? (w >> 16) : (w & 0xFFFFu);
  const float f16 = f16_bits_to_f32(h);
  const float bf = __uint_as_float(h << 16);
  return dtype == W4_F32 ? __uint_as_float(w) : (dtype == W4_F16 ? f16 : bf);
}

// s_waitcnt immediate (gfx9 encoding): at most `vm` vector-memory operations
// outstanding, every LDS operation done, export count left free.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

// Tile order.  Workgroups are dealt round-robin to the 8 XCDs (each with its
// own L2) in launch order.  They are renumbered so that each XCD receives a
// contiguous range of tile numbers t, and t runs through the (m, n) tiles in
// groups of GM m-tiles: the workgroups one XCD runs together cover a patch of
// GM m-tiles x (their number / GM) n-tiles, so each activation and weight
// strip they read is shared through that L2 by several of them.  GM balances
// the patch's bytes per K step: an m-tile of R rows reads R x 128 activation
// bytes, an n-tile of C columns C x 64 weight bytes.  The K split index is
// outermost.  Any permutation is correct; this one only changes locality.
constexpr int kXcds = 8;
template <int GM = 8>
__device__ __forceinline__ void tile_of_block(int& bx, int& by, int& bz) {
  constexpr int kGroupM = GM;
  const int gx = gridDim.x, gy = gridDim.y;
  const int total = gx * gy * gridDim.z;
  const int b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int xcd = b % kXcds, idx = b / kXcds;
  const int per = total / kXcds, rem = total % kXcds;
  const int t = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  bz = t / (gx * gy);
  const int mn = t - bz * gx * gy;
  const int in_group = kGroupM * gy;              // tiles per group of kGroupM m-tiles
  const int group = mn / in_group;
  const int first_m = group * kGroupM;
  const int size_m = gx - first_m < kGroupM ? gx - first_m : kGroupM;
  const int r = mn - group * in_group;
  bx = first_m + r % size_m;
  by = r / size_m;
}

// LDS layout of an activation tile: rows of 128 k (ROWB bytes), unpadded;
// 16-byte chunk c of row R is stored in slot c ^ swz(R), where swz depends on
// R mod 16 only.  A wave's fragment read takes one chunk of 16 consecutive
// rows; the swizzle makes those 16 chunks cover 64 distinct 4-byte banks, and
// every 8 of them 32 distinct banks.
template <int EB>
__device__ __forceinline__ int lds_swizzle(int row) {
  return EB == 1 ? ((row & 7) ^ ((row >> 3) & 1)) : (row & 15);
}

// 16 bytes per lane from a buffer straight into LDS (lane l writes bytes
// [16 l, 16 l + 16) from the wave-uniform base `lds`).  Kept out of kernel
// bodies: the host-side pass of a kernel template that calls the builtin
// directly emits no launch stub.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)off, 0, 0, 0);
}

// MFMAs per 16 x 128 weight block (int8: 2, fp8: 1, fp16 / bf16: 4).
template <int OP>
constexpr int kMfmaPerBlock = OP == OP_I8 ? 2 : (OP == OP_FP8 ? 1 : 4);

// Operand words expand_weights produces per block (8-bit: 8, 16-bit: 16).
template <int OP>
constexpr int kExpandedWords = OpTraits<OP>::kElemBytes * 8;

// Ties N words to an empty asm statement with a memory clobber: everything
// that computes them is scheduled before it, every memory access after it.
template <int N>
__device__ __forceinline__ void pin_words(uint32_t* e) {
  static_assert(N % 8 == 0, "pinned in groups of 8");
#pragma unroll
  for (int i = 0; i < N; i += 8)
    asm volatile("" : "+v"(e[i]), "+v"(e[i + 1]), "+v"(e[i + 2]), "+v"(e[i + 3]), "+v"(e[i + 4]),
                 "+v"(e[i + 5]), "+v"(e[i + 6]), "+v"(e[i + 7])::"memory");
}


// Block-wide barrier that first waits until at most VM of this wave's vector
// memory operations are outstanding.  The direct-to-LDS loads that fill a
// tile stage are vector memory operations the compiler does not order against
// LDS reads, so the wait is explicit; the empty asm statements keep every
// memory access on its side of the barrier.
template <int VM>
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace w4
