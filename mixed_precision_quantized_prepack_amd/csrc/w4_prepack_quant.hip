// Weight prepack (PB-v1) and dynamic per-token activation quantisation.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

// ---------------------------------------------------------------------------
// Prepack.  Machete README, "API": the weight is reordered once into the
// matrix-core operand layout before any GEMM; Machete W4A8 PR summary: the
// reorder only moves data, so it is the same for every 4-bit weight type.
//
// One thread per (n, kb, kq): it reads the 16 logical bytes holding k in
// [128 kb + 32 kq, +32) of row n (coalesced along the row), permutes the
// nibbles inside each 32-bit word and writes the 16 bytes of PB-v1 lane
// 16 kq + n%16 of block (n/16, kb).  Word-internal orders:
//   logical: nibble i (bits 4i) = k-offset i
//   I8     : byte b = k-offset b (low nibble) | k-offset 4+b (high nibble)
//   F16    : low half = k-offsets 0,2,4,6 ; high half = 1,3,5,7 (ExLlama)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t spread_nibbles_to_bytes(uint32_t x16) {
  // nibble b of a 16-bit value -> bits 8b..8b+3
  uint32_t x = (x16 | (x16 << 8)) & 0x00FF00FFu;
  return (x | (x << 4)) & 0x0F0F0F0Fu;
}
__device__ __forceinline__ uint32_t gather_byte_nibbles(uint32_t x) {
  // low nibble of byte b (x & 0x0F0F0F0F) -> nibble b of a 16-bit value
  x = (x | (x >> 4)) & 0x00FF00FFu;
  return (x | (x >> 8)) & 0x0000FFFFu;
}
__device__ __forceinline__ uint32_t reorder_i8(uint32_t w) {
  return spread_nibbles_to_bytes(w & 0xFFFFu) | (spread_nibbles_to_bytes(w >> 16) << 4);
}
__device__ __forceinline__ uint32_t reorder_f16(uint32_t w) {
  return gather_byte_nibbles(w & 0x0F0F0F0Fu) | (gather_byte_nibbles((w >> 4) & 0x0F0F0F0Fu) << 16);
}

template <bool F16CLASS>
__global__ __launch_bounds__(256) void w4_prepack_kernel(const uint4* __restrict__ in,
                                                         uint4* __restrict__ out, int64_t N,
                                                         int64_t K) {
  const int64_t units_per_row = K / 32;
  const int64_t total = N * units_per_row;
  const int64_t KB = K / 128;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = u / units_per_row;
    const int64_t rem = u - n * units_per_row;
    const int64_t kb = rem >> 2;
    const int kq = (int)(rem & 3);
    uint4 v = in[u];
    if (F16CLASS) {
      v.x = reorder_f16(v.x); v.y = reorder_f16(v.y); v.z = reorder_f16(v.z); v.w = reorder_f16(v.w);
    } else {
      v.x = reorder_i8(v.x); v.y = reorder_i8(v.y); v.z = reorder_i8(v.z); v.w = reorder_i8(v.w);
    }
    const int64_t block = (n >> 4) * KB + kb;
    const int lane = kq * 16 + (int)(n & 15);
    out[block * 64 + lane] = v;
  }
}

hipError_t launch_prepack(const void* w_logical, void* w_packed, int64_t N, int64_t K, int operand,
                          hipStream_t stream) {
  const int64_t total = N * (K / 32);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > (1 << 20)) blocks = 1 << 20;  // grid-stride beyond this
  if (operand == W4_OPERAND_F16)
    hipLaunchKernelGGL(w4_prepack_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4*)w_logical, (uint4*)w_packed, N, K);
  else
    hipLaunchKernelGGL(w4_prepack_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4*)w_logical, (uint4*)w_packed, N, K);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dynamic per-token quantisation.  "[ Kernel ] Enable Dynamic Per Token fp8",
// summary and review discussion: one scale per row computed at run time from
// the row's absolute maximum.
//
// One workgroup per row (256 threads, or 1024 when there are few rows so that
// a single row is not latency bound).  Each thread keeps up to kMaxChunks
// 16-byte chunks (8 elements) of the row in registers, so the row is read from
// HBM once: pass 1 takes the absolute maximum, a wave reduction plus an LDS
// exchange gives the row maximum, pass 2 forms the quotients and stores the
// codes.  Longer rows re-read their tail in pass 2.
//
// Quotients x / s must be the correctly rounded fp32 division.  They are
// formed from one correctly rounded reciprocal per row, y = RN(1/s):
// q = RN(x * y), the exact residual r = fma(-q, s, x), and RN(q + r * y), which
// equals RN(x / s) by Markstein's theorem (y within half an ulp of 1/s, q
// within one ulp of x/s, r exact; no overflow or underflow).  Rows whose scale
// is too small for that (bf16 inputs near the bottom of the exponent range)
// use the plain division.
// ---------------------------------------------------------------------------
// Chunks a thread keeps in registers: the launch picks the smallest of
// 4, 8 or 12 that covers the row (a chunk slot past the row still costs an
// address-pipeline pass, which matters when few rows share a CU).
constexpr int kMaxChunks = 12;

template <int XT>
__device__ __forceinline__ float elem(const uint4& v, int j) {
  const uint32_t w = (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w;
  const uint32_t b = (j & 1) ? (w >> 16) : (w & 0xFFFFu);
  return XT == W4_F16 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
}

template <int XT>
__device__ __forceinline__ float chunk_absmax(float m, const uint4& v) {
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(elem<XT>(v, j)));
  return m;
}

// correctly rounded x / s given y = RN(1 / s) (see above).  The sum q + r*y
// of a zero quotient is +0 even for x = -0, so the sign is taken from x (with
// s > 0 the quotient always has the sign of x).
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q = x * y;
  const float r = fmaf(-q, s, x);
  return copysignf(fmaf(r, y, q), x);
}

template <int XT, int QT, bool FAST>
__device__ __forceinline__ uint2 quant_chunk(const uint4& v, float s, float y) {
  uint32_t out[2];
  if (QT == W4_I8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = elem<XT>(v, 4 * h + j);
        float q = rintf(FAST ? div_rn(x, s, y) : x / s);
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        word |= ((uint32_t)(int)q & 0xFFu) << (8 * j);
      }
      out[h] = word;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = elem<XT>(v, 4 * h + j);
        q[j] = fminf(fmaxf(FAST ? div_rn(x, s, y) : x / s, -448.0f), 448.0f);
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
      out[h] = (uint32_t)word;
    }
  }
  return make_uint2(out[0], out[1]);
}

// The row's chunks are read and written with buffer operations: chunk
// indices past the row get an out-of-range offset, which loads zeros (no
// effect on the maximum) and drops the store, so no load or store sits in a
// branch (a branch around a load makes the compiler wait for it on the spot).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kRowOutOfRange = 0x80000000u;

template <int XT, int QT, int THREADS, int CH>
__global__ __launch_bounds__(THREADS) void w4_quant_kernel(const uint16_t* __restrict__ x,
                                                           uint8_t* __restrict__ xq,
                                                           float* __restrict__ scales, int64_t K) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nchunks = (int)(K / 8);
  const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + row * K, K * 2);
  const __amdgpu_buffer_rsrc_t rq = row_rsrc(xq + row * K, K);
  auto load = [&](int idx) -> uint4 {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
        rx, (int)(idx < nchunks ? (uint32_t)idx * 16u : kRowOutOfRange), 0, 0);
    return make_uint4(w.x, w.y, w.z, w.w);
  };
  auto store = [&](int idx, uint2 q) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{q.x, q.y}, rq,
                                          (int)(idx < nchunks ? (uint32_t)idx * 8u : kRowOutOfRange), 0, 0);
  };

  uint4 v[CH];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = load(c * THREADS + tid);
#pragma unroll
  for (int c = 0; c < CH; ++c) amax = chunk_absmax<XT>(amax, v[c]);
  for (int idx = CH * THREADS + tid; idx < nchunks; idx += THREADS) amax = chunk_absmax<XT>(amax, load(idx));

  // row maximum: wave butterfly, then one value per wave through LDS
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  __shared__ float wave_max[THREADS / 64];
  if ((tid & 63) == 0) wave_max[tid >> 6] = amax;
  __syncthreads();
  amax = wave_max[0];
#pragma unroll
  for (int w = 1; w < THREADS / 64; ++w) amax = fmaxf(amax, wave_max[w]);

  const float qmax = (QT == W4_I8) ? 127.0f : 448.0f;
  const float s = amax / qmax;
  if (tid == 0) scales[row] = s;
  if (s == 0.0f) {
    for (int idx = tid; idx < nchunks; idx += THREADS) store(idx, make_uint2(0u, 0u));
    return;
  }
  const float y = 1.0f / s;
  if (s >= 0x1p-100f) {
#pragma unroll
    for (int c = 0; c < CH; ++c) store(c * THREADS + tid, quant_chunk<XT, QT, true>(v[c], s, y));
    for (int idx = CH * THREADS + tid; idx < nchunks; idx += THREADS)
      store(idx, quant_chunk<XT, QT, true>(load(idx), s, y));
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) store(c * THREADS + tid, quant_chunk<XT, QT, false>(v[c], s, y));
    for (int idx = CH * THREADS + tid; idx < nchunks; idx += THREADS)
      store(idx, quant_chunk<XT, QT, false>(load(idx), s, y));
  }
}

template <int THREADS, int CH>
static void launch_quant_t(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                           int64_t K, hipStream_t stream) {
  const dim3 grid((unsigned)M), block(THREADS);
  const uint16_t* xp = (const uint16_t*)x;
  uint8_t* qp = (uint8_t*)xq;
  if (x_dtype == W4_F16 && q_dtype == W4_I8)
    hipLaunchKernelGGL((w4_quant_kernel<W4_F16, W4_I8, THREADS, CH>), grid, block, 0, stream, xp, qp, scales, K);
  else if (x_dtype == W4_F16)
    hipLaunchKernelGGL((w4_quant_kernel<W4_F16, W4_FP8_E4M3, THREADS, CH>), grid, block, 0, stream, xp, qp, scales,
                       K);
  else if (q_dtype == W4_I8)
    hipLaunchKernelGGL((w4_quant_kernel<W4_BF16, W4_I8, THREADS, CH>), grid, block, 0, stream, xp, qp, scales, K);
  else
    hipLaunchKernelGGL((w4_quant_kernel<W4_BF16, W4_FP8_E4M3, THREADS, CH>), grid, block, 0, stream, xp, qp,
                       scales, K);
}

template <int THREADS>
static void launch_quant_c(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                           int64_t K, hipStream_t stream) {
  const int64_t per_thread = (K / 8 + THREADS - 1) / THREADS;
  if (per_thread <= 4)
    launch_quant_t<THREADS, 4>(x, x_dtype, xq, q_dtype, scales, M, K, stream);
  else if (per_thread <= 8)
    launch_quant_t<THREADS, 8>(x, x_dtype, xq, q_dtype, scales, M, K, stream);
  else
    launch_quant_t<THREADS, kMaxChunks>(x, x_dtype, xq, q_dtype, scales, M, K, stream);
}

hipError_t launch_quant(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                        int64_t K, hipStream_t stream) {
  // few rows: a whole CU per row
  if (M <= 512 && K >= 8 * 1024)
    launch_quant_c<1024>(x, x_dtype, xq, q_dtype, scales, M, K, stream);
  else
    launch_quant_c<256>(x, x_dtype, xq, q_dtype, scales, M, K, stream);
  return hipGetLastError();
}

}  // namespace w4
