// Weight prepack (PB-v1) and dynamic per-token activation quantisation.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {

// ---------------------------------------------------------------------------
// Prepack.  Machete README, "API": the weight is reordered once into the
// matrix-core operand layout before any GEMM; Machete W4A8 PR summary: the
// reorder only moves data, so it is the same for every 4-bit weight type.
//
// One thread per PB-v1 lane slot, 64 consecutive threads per 1 KiB block
// (the writes of a wave are one contiguous KiB): thread u fills lane
// l = u mod 64 = 16 kq + r of block u / 64 = (n / 16, kb), reading the 16
// logical bytes that hold k in [128 kb + 32 kq, +32) of row n = 16 nb + r
// (per wave, 64 contiguous bytes of each of 16 rows; the next wave reads the
// rest of those lines), and permutes the nibbles inside each 32-bit word.
// Word-internal orders:
//   logical: nibble i (bits 4i) = k-offset i
//   I8     : byte b = k-offset b (low nibble) | k-offset 4+b (high nibble)
//   F16    : low half = k-offsets 0,2,4,6 ; high half = 1,3,5,7 (ExLlama)
//
// The importer of ExLlama-shuffled int32 words [N, K/8] (W4A16 page,
// docstring of the skinny-format kernel) runs the same kernel: 16 bytes of
// a source row are the 32 k of one PB-v1 lane slot as well, and its words
// are in the F16 order already (identity), while reorder_i8 of an F16-order
// word is its logical word, so I8 takes reorder_i8 twice.
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

template <bool F16CLASS, bool EXLLAMA>
__global__ __launch_bounds__(256) void w4_prepack_kernel(const uint4* __restrict__ in,
                                                         uint4* __restrict__ out, int64_t N,
                                                         int64_t K) {
  const int64_t units_per_row = K / 32;
  const int64_t total = N * units_per_row;
  const int64_t KB = K / 128;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    // block < N K / 2048 < 2^32 (the host rejects larger weights)
    const uint32_t block = (uint32_t)(u >> 6);
    const int lane = (int)(u & 63);
    const int64_t nb = block / (uint32_t)KB, kb = block - (uint32_t)nb * (uint32_t)KB;
    const int64_t n = nb * 16 + (lane & 15);
    const int kq = lane >> 4;
    uint4 v = in[n * units_per_row + kb * 4 + kq];
    if (EXLLAMA && !F16CLASS) {
      v.x = reorder_i8(v.x); v.y = reorder_i8(v.y); v.z = reorder_i8(v.z); v.w = reorder_i8(v.w);
    }
    if (F16CLASS && !EXLLAMA) {
      v.x = reorder_f16(v.x); v.y = reorder_f16(v.y); v.z = reorder_f16(v.z); v.w = reorder_f16(v.w);
    } else if (!F16CLASS) {
      v.x = reorder_i8(v.x); v.y = reorder_i8(v.y); v.z = reorder_i8(v.z); v.w = reorder_i8(v.w);
    }
    out[u] = v;
  }
}

hipError_t launch_prepack(const void* w_in, void* w_packed, int64_t N, int64_t K, int operand, bool exllama,
                          hipStream_t stream) {
  const int64_t total = N * (K / 32);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > (1 << 20)) blocks = 1 << 20;  // grid-stride beyond this
  const dim3 g((unsigned)blocks), b(threads);
  const uint4* in = (const uint4*)w_in;
  uint4* out = (uint4*)w_packed;
  if (operand == W4_OPERAND_F16 && exllama)
    hipLaunchKernelGGL((w4_prepack_kernel<true, true>), g, b, 0, stream, in, out, N, K);
  else if (operand == W4_OPERAND_F16)
    hipLaunchKernelGGL((w4_prepack_kernel<true, false>), g, b, 0, stream, in, out, N, K);
  else if (exllama)
    hipLaunchKernelGGL((w4_prepack_kernel<false, true>), g, b, 0, stream, in, out, N, K);
  else
    hipLaunchKernelGGL((w4_prepack_kernel<false, false>), g, b, 0, stream, in, out, N, K);
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
// codes.  Longer rows re-read their tail in pass 2.  The chunk coder
// (elem, chunk_absmax, div_rn, quant_chunk) is in w4_device.h.
//
// Chunks a thread keeps in registers: the launch picks the smallest of
// 4, 8 or 12 that covers the row (a chunk slot past the row still costs an
// address-pipeline pass, which matters when few rows share a CU), and at
// most 4 in 1024-thread workgroups.
constexpr int kMaxChunks = 12;

// ---------------------------------------------------------------------------
// Fused RMSNorm.  "[ Kernel ] Enable Dynamic Per Token fp8", review
// discussion: per-token scales make it easy to fuse the preceding RMSNorm
// with the quantisation.  The fused operation returns what the RMSNorm
// (output in the activation dtype) followed by the quantisation above would:
//   ss = sum_k x^2 (rounded once to fp64), r = fp32(1 / sqrt(ss / K + eps))
//   (fp64 arithmetic), y = dtype(fp32(fp32(x * r) * gamma)), then quantise y.
// The sum of squares decides integer codes, so r must be the one its exact
// sum gives.  Each square is exact in fp64.  Fast path: every thread sums its
// n terms with fp64 FMAs; the terms are positive, so the result is within
// n * 2^-53 (relative) of their exact sum, and the threads' sums are combined
// as unevaluated pairs hi + lo (error-free two-sums).  r is computed from both
// ends of that interval through the same monotone fp64 steps, widened by a
// few ulps; when both round to the same fp32 value, that value is r.  Else
// (about one row in 2^22) the exact path re-sums the row's squares as pairs,
// with an error-free two-sum per term (within ~2^-100 of the exact sum), so
// that hi is the sum rounded once.
// ---------------------------------------------------------------------------
struct DD {
  double hi, lo;
};

// hi + lo += p, with the rounding error of hi + p kept exactly (two-sum)
__device__ __forceinline__ void dd_add_term(DD& a, double p) {
  const double s = a.hi + p;
  const double bp = s - a.hi;
  const double e = (a.hi - (s - bp)) + (p - bp);
  a.hi = s;
  a.lo += e;
}

// (a.hi + a.lo) + (b.hi + b.lo), renormalised so that hi is the pair rounded
// once.  Symmetric in a and b, so both lanes of a butterfly agree.
__device__ __forceinline__ DD dd_add(const DD& a, const DD& b) {
  const double s = a.hi + b.hi;
  const double bp = s - a.hi;
  double e = (a.hi - (s - bp)) + (b.hi - bp);
  e += a.lo + b.lo;
  const double hi = s + e;
  return DD{hi, e - (hi - s)};
}

template <int XT>
__device__ __forceinline__ void dd_add_chunk(DD& a, const uint4& v) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const double x = (double)elem<XT>(v, j);
    dd_add_term(a, x * x);   // exact: at most 22 significant bits
  }
}

// 1 / sqrt(ss / K + eps) in fp64: monotone (non-increasing) in ss
__device__ __forceinline__ double rms_recip(double ss, int64_t K, float eps) {
  return 1.0 / sqrt(ss / (double)K + (double)eps);
}

template <int XT>
__device__ __forceinline__ uint32_t to_dtype_bits(float v) {
  return XT == W4_F16 ? (uint32_t)f32_to_f16_bits(v) : (uint32_t)f32_to_bf16_bits(v);
}

// y = dtype(fp32(fp32(x * r) * gamma)) for the 8 elements of a chunk, packed
// in the chunk layout elem() reads.  The fp32 product passes through an empty
// asm statement: otherwise the compiler fuses the multiply with the fp16
// conversion (v_fma_mixlo_f16), which rounds the exact product once instead
// of rounding the fp32 product, and differs from it at fp16 ties.
template <int XT>
__device__ __forceinline__ uint4 norm_chunk(const uint4& x, const uint4& g, float r) {
  uint32_t w[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float y0 = (elem<XT>(x, 2 * h) * r) * elem<XT>(g, 2 * h);
    float y1 = (elem<XT>(x, 2 * h + 1) * r) * elem<XT>(g, 2 * h + 1);
    asm volatile("" : "+v"(y0), "+v"(y1));
    w[h] = to_dtype_bits<XT>(y0) | (to_dtype_bits<XT>(y1) << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The row's chunks are read and written with buffer operations: chunk
// indices past the row get an out-of-range offset, which loads zeros (no
// effect on the maximum) and drops the store, so no load or store sits in a
// branch (a branch around a load makes the compiler wait for it on the spot).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kRowOutOfRange = 0x80000000u;

// Where a row's scale comes from.  Per-token: the row's own maximum.  The
// per-tensor scale ("[ Kernel ] Enable Dynamic Per Token fp8", results and
// review discussion: one scale for the whole tensor, computed at run time)
// takes three launches, since no row can be coded before every row has been
// read: the row maxima (written to scales[row], no codes), their maximum
// (w4_tensor_scale_kernel, which writes the tensor's scale to every
// scales[row]), then the codes with the scale read from scales[row].
enum { kScaleRow = 0, kScaleRowMaxOnly = 1, kScaleGiven = 2 };

// 256-thread int8 workgroups: three per CU (at most 168 VGPRs); the fp8
// coder needs more registers than that with 12 chunks per thread.
template <int XT, int QT, int THREADS, int CH, bool NORM, int SC>
__global__ __launch_bounds__(THREADS, (THREADS == 256 && QT == W4_I8) ? 3 : 1) void w4_quant_kernel(const uint16_t* __restrict__ x,
                                                           uint8_t* __restrict__ xq,
                                                           float* __restrict__ scales, int64_t K,
                                                           const uint16_t* __restrict__ gamma, float eps,
                                                           int exact_sum) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nchunks = (int)(K / 8);
  const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + row * K, K * 2);
  const __amdgpu_buffer_rsrc_t rq = row_rsrc(xq + row * K, K);
  const __amdgpu_buffer_rsrc_t rg = row_rsrc(gamma, NORM ? K * 2 : 0);
  auto load_raw = [&](const __amdgpu_buffer_rsrc_t& rsrc, int idx) -> uint4 {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
        rsrc, (int)(idx < nchunks ? (uint32_t)idx * 16u : kRowOutOfRange), 0, 0);
    return make_uint4(w.x, w.y, w.z, w.w);
  };
  __shared__ float wave_max[THREADS / 64];
  __shared__ DD wave_ss[NORM ? THREADS / 64 : 1];
  // fused RMSNorm: the row's scale factor, computed once the row is loaded
  float r = 1.0f;
  // a chunk of the quantiser's input: x itself, or the normalised x
  auto load = [&](int idx) -> uint4 {
    const uint4 v = load_raw(rx, idx);
    if constexpr (NORM) return norm_chunk<XT>(v, load_raw(rg, idx), r);
    return v;
  };
  auto store = [&](int idx, uint2 q) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{q.x, q.y}, rq,
                                          (int)(idx < nchunks ? (uint32_t)idx * 8u : kRowOutOfRange), 0, 0);
  };

  uint4 v[CH];
  float amax = 0.0f;
  // a given scale is read before the row, so its load is in flight with them
  const float s_given = SC == kScaleGiven ? scales[row] : 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) v[c] = load_raw(rx, c * THREADS + tid);
  if constexpr (NORM) {
    // pairs summed over the workgroup: wave butterfly, then the waves in order
    auto block_sum = [&](DD a) -> DD {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1)
        a = dd_add(a, DD{__shfl_xor(a.hi, off, 64), __shfl_xor(a.lo, off, 64)});
      __syncthreads();   // the previous sum's readers are done with wave_ss
      if ((tid & 63) == 0) wave_ss[tid >> 6] = a;
      __syncthreads();
      a = wave_ss[0];
#pragma unroll
      for (int w = 1; w < THREADS / 64; ++w) a = dd_add(a, wave_ss[w]);
      return a;
    };
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double xv = (double)elem<XT>(v[c], j);
        acc = fma(xv, xv, acc);
      }
    for (int idx = CH * THREADS + tid; idx < nchunks; idx += THREADS) {
      const uint4 t = load_raw(rx, idx);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double xv = (double)elem<XT>(t, j);
        acc = fma(xv, xv, acc);
      }
    }
    const DD ss = block_sum(DD{acc, 0.0});
    // a thread sums at most n terms; the bound also covers the roundings of
    // the pair sums and of ss * (1 +- rho)
    const int64_t n = 8 * (((int64_t)nchunks + THREADS - 1) / THREADS);
    const double rho = (double)(n + 8) * 0x1p-53;
    const float r_lo = (float)(rms_recip(ss.hi * (1.0 + rho), K, eps) * (1.0 - 0x1p-50));
    const float r_hi = (float)(rms_recip(ss.hi * (1.0 - rho), K, eps) * (1.0 + 0x1p-50));
    if (r_lo == r_hi && !exact_sum) {
      r = r_lo;
    } else {
      DD e{0.0, 0.0};
      // the row is read again (rather than taken from the chunks in
      // registers, which the compiler would then keep in twice the registers)
      for (int idx = tid; idx < nchunks; idx += THREADS) dd_add_chunk<XT>(e, load_raw(rx, idx));
      e = block_sum(dd_add(DD{0.0, 0.0}, e));
      r = (float)rms_recip(e.hi, K, eps);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = norm_chunk<XT>(v[c], load_raw(rg, c * THREADS + tid), r);
  }
  if constexpr (SC != kScaleGiven) {
#pragma unroll
    for (int c = 0; c < CH; ++c) amax = chunk_absmax<XT>(amax, v[c]);
    for (int idx = CH * THREADS + tid; idx < nchunks; idx += THREADS) amax = chunk_absmax<XT>(amax, load(idx));

    // row maximum: wave butterfly, then one value per wave through LDS
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((tid & 63) == 0) wave_max[tid >> 6] = amax;
    __syncthreads();
    amax = wave_max[0];
#pragma unroll
    for (int w = 1; w < THREADS / 64; ++w) amax = fmaxf(amax, wave_max[w]);
    if constexpr (SC == kScaleRowMaxOnly) {
      if (tid == 0) scales[row] = amax;
      return;
    }
  }

  const float qmax = (QT == W4_I8) ? 127.0f : 448.0f;
  const float s = SC == kScaleGiven ? s_given : amax / qmax;
  if (SC == kScaleRow && tid == 0) scales[row] = s;
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

// Per-token quantisation of a few long rows: P workgroups per row, so that a
// batch of a few tokens keeps P CUs per row busy instead of one.  Every
// workgroup finds the maximum of the whole row (its re-reads of the row hit
// the L2; the maximum is exact in any order) and codes its own P-th of the
// chunks.  Scale and codes are those of w4_quant_kernel; part 0 writes the
// scale.
#ifndef W4_QUANT_PARTS_MAX
#define W4_QUANT_PARTS_MAX 16
#endif
template <int XT, int QT>
__global__ __launch_bounds__(256) void w4_quant_parts_kernel(const uint16_t* __restrict__ x,
                                                             uint8_t* __restrict__ xq,
                                                             float* __restrict__ scales, int64_t K) {
  constexpr int T = 256;
  constexpr int B = 8;   // chunk loads per thread in flight in the maximum pass
  const int64_t row = blockIdx.y;
  const int part = blockIdx.x, parts = gridDim.x;
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
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{q.x, q.y}, rq, (int)((uint32_t)idx * 8u), 0, 0);
  };
  __shared__ float wave_max[T / 64];
  // the whole row's maximum (chunks past the row read zero)
  float amax = 0.0f;
  for (int base = 0; base < nchunks; base += B * T) {
    uint4 v[B];
#pragma unroll
    for (int c = 0; c < B; ++c) v[c] = load(base + c * T + tid);
#pragma unroll
    for (int c = 0; c < B; ++c) amax = chunk_absmax<XT>(amax, v[c]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) wave_max[tid >> 6] = amax;
  __syncthreads();
  amax = wave_max[0];
#pragma unroll
  for (int w = 1; w < T / 64; ++w) amax = fmaxf(amax, wave_max[w]);

  const float s = amax / ((QT == W4_I8) ? 127.0f : 448.0f);
  if (part == 0 && tid == 0) scales[row] = s;
  const int c0 = (int)((int64_t)nchunks * part / parts);
  const int c1 = (int)((int64_t)nchunks * (part + 1) / parts);
  if (s == 0.0f) {
    for (int idx = c0 + tid; idx < c1; idx += T) store(idx, make_uint2(0u, 0u));
    return;
  }
  const float y = 1.0f / s;
  if (s >= 0x1p-100f) {
    for (int idx = c0 + tid; idx < c1; idx += T) store(idx, quant_chunk<XT, QT, true>(load(idx), s, y));
  } else {
    for (int idx = c0 + tid; idx < c1; idx += T) store(idx, quant_chunk<XT, QT, false>(load(idx), s, y));
  }
}

// The tensor's scale from its row maxima (held in scales[0, M)):
// s = fp32(max_m scales[m] / qmax), written to every scales[m].  One
// workgroup; each thread writes only the entries it has read, after the
// barrier that every read precedes.
template <int QT>
__global__ __launch_bounds__(1024) void w4_tensor_scale_kernel(float* __restrict__ scales, int64_t M) {
  const int tid = threadIdx.x;
  __shared__ float wave_max[16];
  float m = 0.0f;
  for (int64_t i = tid; i < M; i += 1024) m = fmaxf(m, scales[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((tid & 63) == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  m = wave_max[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) m = fmaxf(m, wave_max[w]);
  const float s = m / ((QT == W4_I8) ? 127.0f : 448.0f);
  for (int64_t i = tid; i < M; i += 1024) scales[i] = s;
}

template <int THREADS, int CH, bool NORM, int SC = kScaleRow>
static void launch_quant_t(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                           int64_t K, const void* gamma, float eps, int exact, hipStream_t stream) {
  const dim3 grid((unsigned)M), block(THREADS);
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* gp = (const uint16_t*)gamma;
  uint8_t* qp = (uint8_t*)xq;
  if (x_dtype == W4_F16 && q_dtype == W4_I8)
    hipLaunchKernelGGL((w4_quant_kernel<W4_F16, W4_I8, THREADS, CH, NORM, SC>), grid, block, 0, stream, xp, qp,
                       scales, K, gp, eps, exact);
  else if (x_dtype == W4_F16)
    hipLaunchKernelGGL((w4_quant_kernel<W4_F16, W4_FP8_E4M3, THREADS, CH, NORM, SC>), grid, block, 0, stream, xp, qp,
                       scales, K, gp, eps, exact);
  else if (q_dtype == W4_I8)
    hipLaunchKernelGGL((w4_quant_kernel<W4_BF16, W4_I8, THREADS, CH, NORM, SC>), grid, block, 0, stream, xp, qp,
                       scales, K, gp, eps, exact);
  else
    hipLaunchKernelGGL((w4_quant_kernel<W4_BF16, W4_FP8_E4M3, THREADS, CH, NORM, SC>), grid, block, 0, stream, xp,
                       qp, scales, K, gp, eps, exact);
}

// 1024-thread workgroups keep at most 4 chunks per thread (128 VGPRs per
// thread at that size; 8 or 12 chunks would spill), longer rows re-read
// their tail.
template <int THREADS, bool NORM, int SC>
static void launch_quant_c(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                           int64_t K, const void* gamma, float eps, int exact, hipStream_t stream) {
  const int64_t per_thread = (K / 8 + THREADS - 1) / THREADS;
  if constexpr (THREADS > 256)
    launch_quant_t<THREADS, 4, NORM, SC>(x, x_dtype, xq, q_dtype, scales, M, K, gamma, eps, exact, stream);
  else if (per_thread <= 4)
    launch_quant_t<THREADS, 4, NORM, SC>(x, x_dtype, xq, q_dtype, scales, M, K, gamma, eps, exact, stream);
  else if (per_thread <= 8)
    launch_quant_t<THREADS, 8, NORM, SC>(x, x_dtype, xq, q_dtype, scales, M, K, gamma, eps, exact, stream);
  else
    launch_quant_t<THREADS, kMaxChunks, NORM, SC>(x, x_dtype, xq, q_dtype, scales, M, K, gamma, eps, exact,
                                                  stream);
}

template <bool NORM, int SC = kScaleRow>
static void launch_quant_n(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                           int64_t K, const void* gamma, float eps, int exact, hipStream_t stream) {
  // few rows: a whole CU per row
  if (M <= 512 && K >= 8 * 1024)
    launch_quant_c<1024, NORM, SC>(x, x_dtype, xq, q_dtype, scales, M, K, gamma, eps, exact, stream);
  else
    launch_quant_c<256, NORM, SC>(x, x_dtype, xq, q_dtype, scales, M, K, gamma, eps, exact, stream);
}

hipError_t launch_quant(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                        int64_t K, hipStream_t stream) {
  // a few long rows: several workgroups per row (P = 16 rows' worth of CUs
  // per row up to M = 16, 4 up to M = 64)
  if (K >= 8192 && M > 0 && M <= 64) {
    const int parts = M <= 16 ? W4_QUANT_PARTS_MAX : 4;
    const dim3 grid((unsigned)parts, (unsigned)M), block(256);
    const uint16_t* xp = (const uint16_t*)x;
    uint8_t* qp = (uint8_t*)xq;
    if (x_dtype == W4_F16 && q_dtype == W4_I8)
      hipLaunchKernelGGL((w4_quant_parts_kernel<W4_F16, W4_I8>), grid, block, 0, stream, xp, qp, scales, K);
    else if (x_dtype == W4_F16)
      hipLaunchKernelGGL((w4_quant_parts_kernel<W4_F16, W4_FP8_E4M3>), grid, block, 0, stream, xp, qp, scales, K);
    else if (q_dtype == W4_I8)
      hipLaunchKernelGGL((w4_quant_parts_kernel<W4_BF16, W4_I8>), grid, block, 0, stream, xp, qp, scales, K);
    else
      hipLaunchKernelGGL((w4_quant_parts_kernel<W4_BF16, W4_FP8_E4M3>), grid, block, 0, stream, xp, qp, scales, K);
    return hipGetLastError();
  }
  launch_quant_n<false>(x, x_dtype, xq, q_dtype, scales, M, K, nullptr, 0.0f, 0, stream);
  return hipGetLastError();
}

hipError_t launch_quant_per_tensor(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                                   int64_t K, hipStream_t stream) {
  launch_quant_n<false, kScaleRowMaxOnly>(x, x_dtype, xq, q_dtype, scales, M, K, nullptr, 0.0f, 0, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (q_dtype == W4_I8)
    hipLaunchKernelGGL(w4_tensor_scale_kernel<W4_I8>, dim3(1), dim3(1024), 0, stream, scales, M);
  else
    hipLaunchKernelGGL(w4_tensor_scale_kernel<W4_FP8_E4M3>, dim3(1), dim3(1024), 0, stream, scales, M);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_quant_n<false, kScaleGiven>(x, x_dtype, xq, q_dtype, scales, M, K, nullptr, 0.0f, 0, stream);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quant(const void* x, int x_dtype, const void* gamma, float eps, void* xq, int q_dtype,
                                float* scales, int64_t M, int64_t K, int exact_sum, hipStream_t stream) {
  launch_quant_n<true>(x, x_dtype, xq, q_dtype, scales, M, K, gamma, eps, exact_sum, stream);
  return hipGetLastError();
}

}  // namespace w4
