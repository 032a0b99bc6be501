// W4A8 / W4A16 GEMM kernels for gfx950.
//
//   out[m,n] = RNE( s_a[m] * sum_g s[n,g] * sum_{k in g} a[m,k] * w[n,k] + bias[n] )
//
// (Machete README, "Overview"; "support W4A8 Marlin kernel" for the
// per-channel / per-group W4A8 variants; the rdna_hybrid_w4a16 API page for
// the W4A16 zero-point form (c - z) * s.)
//
// Two kernels share the operand expansion and the MFMA step:
//   * w4_gemm_skinny: M <= 16.  The weight stream is the whole cost, so one
//     wave walks a 16-column strip of W over a contiguous K range with wide
//     (16-byte) loads; the waves of a workgroup split K and are summed through
//     LDS in a fixed order.
//   * w4_gemm_tiled: larger M.  A BM x BN output tile per workgroup; the
//     activation tile of each 128-deep K step is staged in LDS (double
//     buffered) and shared by the four waves, each of which streams its own
//     weight blocks from memory.  Few tiles -> K is split across workgroups
//     and a second kernel sums the partial tiles in a fixed order.
//
// Matrix-core mapping (one PB-v1 block = 16 n x 128 k):
//   MFMA operand A = weights, lane l supplies row n = l%16 and the 32 k of
//   lane group l/16; operand B = activations, lane l supplies row m = l%16
//   with the same k set.  D element i of lane l is (n = 4*(l/16)+i, m = l%16).
//   int8 : 2 x v_mfma_i32_16x16x64_i8   per block (weights as 16*w)
//   fp8  : 1 x v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3 x e4m3, unit scales)
//   fp16 / bf16 : 4 x v_mfma_f32_16x16x32_{f16,bf16}
// Group-128 problems restart the block accumulator every block (one block is
// one group) and fold it into an fp32 total with the group scale.
#include <type_traits>

#include "w4_gemm_common.h"

namespace w4 {

// ===========================================================================
// Small-M kernel.
// ===========================================================================

// Blocks per batch of the small-M kernel (8-bit / 16-bit operands) and the
// cache-policy bits of its weight loads (2 = non-temporal: the weight stream
// is read once).
#ifndef W4_SKINNY_U8
#define W4_SKINNY_U8 1
#endif
#ifndef W4_SKINNY_U16
#define W4_SKINNY_U16 1
#endif
#ifndef W4_SKINNY_UG1
#define W4_SKINNY_UG1 2   // grouped, one strip per wave
#endif
#ifndef W4_SKINNY_UG2
#define W4_SKINNY_UG2 1   // grouped, two strips per wave
#endif
#ifndef W4_TILED_FOLD_BLOCKS
#define W4_TILED_FOLD_BLOCKS 3
#endif
#ifndef W4_SKINNY_WPOLICY
#define W4_SKINNY_WPOLICY 2
#endif


// Small-M kernel (M <= 16).
//
// Workgroup = S waves over the same NS 16-column strips of W; the K blocks are
// dealt to the waves round-robin (wave w takes blocks w, w+S, ...), so at any
// time a workgroup reads S contiguous KiB of each strip.  A wave multiplies
// each activation fragment with its NS weight blocks (NS strips share the
// fragment, which divides the activation traffic by NS).  Batches of U
// K-blocks are double buffered: the loads of batch i+1 (weights, activations
// and, for groups, the group scales / zero-points) are issued before the
// MFMAs of batch i.  Rows past M and blocks past K are buffer loads with
// out-of-range offsets: they read as zero without memory traffic.  The
// waves' results are summed through LDS in wave order.
//
// Group scales (times 1/16 for int8) and W4A16 zero-point terms are staged
// once per workgroup into an LDS table, group-major ([strip][group][row]),
// while the first batch is in flight: a lane then reads the four values of
// its D rows for a K block with one 16-byte LDS read, instead of a 64-lane
// gather from memory per block (which costs the address pipeline as much as
// the block's weights).  The table's size is set at launch.

// Waves per SIMD the small-M kernel is compiled for (the second launch
// bound): six for grouped 8-bit problems with two strips or staged
// activations, whose eight-wave workgroups then fit three to a CU (at most
// 84 registers, no spills); no bound otherwise (the other forms spill under
// it).
template <int OP, bool GROUPED, int NS, bool ZP, bool QA, bool DA>
constexpr int skinny_min_waves() {
  return (OP == OP_I8 || OP == OP_FP8) && GROUPED && !ZP && !QA && (NS == 2 || DA) ? 6 : 1;
}

template <int OP, bool GROUPED, bool FLIP, int NS, bool PARTIALS, bool ZP, int SG, bool QA, bool PZ = false,
          bool DA = false>
__global__ __launch_bounds__(64 * skinny_max_waves(OP, GROUPED), (skinny_min_waves<OP, GROUPED, NS, ZP, QA, DA>()))
void w4_gemm_skinny(GemmArgs p, int S) {
  using Acc = typename OpTraits<OP>::Acc;
  constexpr int EB = OpTraits<OP>::kElemBytes;
  constexpr int AV = act_vecs<OP>();
  constexpr int U = GROUPED ? (NS == 1 ? W4_SKINNY_UG1 : W4_SKINNY_UG2)
                            : (EB == 1) ? W4_SKINNY_U8 : W4_SKINNY_U16;   // K blocks per batch

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nb0 = (int64_t)blockIdx.x * NS;   // first strip of the workgroup
  const int KB = (int)(p.K >> 7);
  const int r = lane & 15;
  const int kq = lane >> 4;
  constexpr bool partials = PARTIALS;  // verification mode: store group partials
  const int zdt = p.z_dtype;                      // zero-point storage dtype
  static_assert(!ZP || (OP == OP_I8 && FLIP), "zero-points: int8 operand from raw uint4 codes");
  static_assert(SG == 1 || (GROUPED && (OP == OP_F16 || OP == OP_BF16)), "sub-groups: grouped W4A16 only");
  static_assert(!QA || ((OP == OP_I8 || OP == OP_FP8) && !PARTIALS && !ZP && SG == 1),
                "fused quantisation: W4A8 outputs only");
  static_assert(!PZ || ((OP == OP_F16 || OP == OP_BF16) && GROUPED && !PARTIALS && SG == 1),
                "pre-scaled zero-points: grouped W4A16 outputs only");

  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(reinterpret_cast<const uint8_t*>(p.b) + nb0 * KB * 1024, (int64_t)NS * KB * 1024);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, QA ? 0 : p.M * p.K * EB);
  const int sbytes = p.s_dtype == W4_F32 ? 4 : 2;
  // scales are absent (null) in the partials entry points: an empty buffer
  // (a product, not a branch: a branch here would wait for the kernel
  // arguments before anything else is issued)
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.s, (int64_t)(p.s != nullptr) * p.N * p.G * sbytes);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(p.z, p.z ? p.N * p.G * (zdt == W4_F32 ? 4 : 2) : 0);
  const uint32_t w_lane = (uint32_t)lane * 16;
  const uint32_t a_lane = (uint32_t)((r * p.K + kq * 32) * EB);

  Acc acc[NS];
  f32x4 ones = {};
  i32x4 ones_i = {};   // asymmetric int8: 16 * sum(a)
  f32x4 tot[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    acc[j] = Acc{};
    tot[j] = f32x4{};
  }
  // Epilogue inputs, fetched now so the kernel's tail does not wait on memory:
  // the element this thread finalises after the reduction (threads below
  // 256 NS; element t = (strip j, lane l, row i)) and, for bf16 W4A16 per
  // channel, the zero-points of this lane's D rows.
  const int ep_j = threadIdx.x >> 8, ep_l = (threadIdx.x >> 2) & 63, ep_i = threadIdx.x & 3;
  const int64_t ep_m = ep_l & 15;
  const int64_t ep_n = (nb0 + ep_j) * 16 + 4 * (ep_l >> 4) + ep_i;
  const bool ep_in = (int)threadIdx.x < 256 * NS && ep_m < p.M && ep_n < p.N;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.a_scales, p.a_scales ? p.M * 4 : 0);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bias, p.bias ? p.N * 2 : 0);
  const uint32_t ep_s = load_word(rs, p.s_dtype, (uint32_t)ep_n, !GROUPED && ep_in);
  const uint32_t ep_a = load_word(rsa, W4_F32, (uint32_t)ep_m, ep_in && p.a_scales);
  const uint32_t ep_b = load_word(rb, p.out_dtype, (uint32_t)ep_n, ep_in && p.bias);
  // fp16 W4A16 per channel: the zero-point of this lane's operand row
  float zrow[NS];
  if constexpr (OP == OP_F16 && !GROUPED) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const uint32_t zi = (uint32_t)((nb0 + j) * 16 + r) * p.G;
      zrow[j] = p.z ? word_to_f32(load_word(rz, zdt, zi, true), zdt, zi) : 8.0f;
    }
  }
  uint32_t zpc[NS][4];
  if constexpr ((OP == OP_BF16 || ZP) && !GROUPED) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        zpc[j][i] = load_word(rz, zdt, (uint32_t)((nb0 + j) * 16 + 4 * kq + i) * p.G, p.z != nullptr);
  }

  u32x4 wv[2][U][NS];
  u32x4 av[2][U][AV];
  // LDS tables: tsc = group scales (grouped), tz = 128 + z (grouped bf16
  // W4A16), z (grouped fp16 W4A16) or z - 8 (grouped asymmetric int8), each
  // [NS][G][16] fp32.
  constexpr bool kTab = skinny_tables(OP, GROUPED, ZP) > 0;
  extern __shared__ __attribute__((aligned(16))) float skinny_tab[];
  // (each table is followed by a 16-float pad that takes the stores of
  // staging slots past its end)
  float* const tsc = skinny_tab;
  float* const tz = skinny_tab + (GROUPED ? NS * p.G * 16 + 16 : 0);
  // fused quantisation: the codes [M][K] (row-major, as the quantiser writes
  // them) after the tables, then a 32-byte zero pad that rows past M and
  // blocks past K read
  uint8_t* const qcodes =
      reinterpret_cast<uint8_t*>(skinny_tab) + skinny_tables(OP, GROUPED, ZP) * (NS * p.G * 16 + 16) * 4;
  // DA (8-bit activations, not fused; M >= 8): each wave stages its K
  // blocks' 16 x 128 activation bytes in LDS by direct-to-LDS loads of whole
  // rows (8 rows of 128 bytes per load, where a 16-row fragment load from
  // memory touches 16 rows for 64 bytes each: int8 per channel 8192 x 21760
  // at M = 16 19.8 -> 17.8 us), two buffers of U blocks per wave, after the
  // tables (16-byte aligned).  Chunk c of row R is at slot c ^ swz(R), as in
  // the tiled kernel, so the fragment reads are conflict-free.  Below M = 8
  // the loads touch few rows either way, and the LDS round trip cost the fp8
  // kernel 1-2% at M = 1 and 5.
  constexpr bool kDma = DA;
  static_assert(!DA || (EB == 1 && !QA), "staged activations: 8-bit, not fused");
  uint8_t* const stg = reinterpret_cast<uint8_t*>(skinny_tab) +
                       ((skinny_tables(OP, GROUPED, ZP) * (NS * p.G * 16 + 16) * 4 + 15) & ~15);
  uint32_t dma_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * h + lane / 8;
    dma_off[h] = (uint32_t)(row * p.K + (((lane & 7) ^ lds_swizzle<1>(row)) * 16));
  }
  int frag_off[AV];
#pragma unroll
  for (int j = 0; j < AV; ++j) frag_off[j] = r * 128 + (((kq * AV + j) ^ lds_swizzle<1>(r)) * 16);
  auto stage_of = [&](int buf, int u) { return stg + ((wave * 2 + buf) * U + u) * 2048; };
  const uint32_t qpad = (uint32_t)(p.M * p.K);
  __shared__ uint32_t qa_max[QA ? 16 : 1];
  __shared__ float qa_s[QA ? 16 : 1];
  // Fused quantisation: per-token quantisation of the M rows into LDS (the
  // same codes and scales as the quantisation kernel).  The waves split into
  // one group per row (rows past the groups' count loop): a group's threads
  // take 16-byte chunks of its row, a wave maximum and an LDS maximum give
  // the row's absolute maximum, then the chunks are coded (re-read from L2
  // unless the group's one row fitted one round of chunks in registers).
  auto quantise_rows = [&]() {
    constexpr int QC = 8;   // chunks per thread per round
    const int nch = (int)(p.K >> 3);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, p.M * p.K * 2);
    constexpr int QT = OP == OP_I8 ? W4_I8 : W4_FP8_E4M3;
    const float qmax = OP == OP_I8 ? 127.0f : 448.0f;
    const bool f16 = p.x_dtype == W4_F16;
    const int nw = (int)(blockDim.x >> 6);
    const int gw = nw >= p.M ? nw / (int)p.M : 1;    // waves per row
    const int ngr = nw / gw;                          // rows in flight
    const int grp = wave / gw;
    const int Tr = gw * 64;
    const int tr = (wave - grp * gw) * 64 + lane;     // thread within the row's group
    const bool keep = p.M <= ngr && nch <= QC * Tr;
    if (threadIdx.x < 16) qa_max[threadIdx.x] = 0u;
    if (threadIdx.x < 8) reinterpret_cast<uint32_t*>(qcodes + qpad)[threadIdx.x] = 0u;
    __syncthreads();
    auto load_round = [&](int m, int c0, uint4* v) {
#pragma unroll
      for (int i = 0; i < QC; ++i) {
        const int c = c0 + tr + i * Tr;
        const u32x4 w = buffer_load16(rx, c < nch ? (uint32_t)((m * p.K + c * 8) * 2) : kOutOfRange);
        v[i] = make_uint4(w.x, w.y, w.z, w.w);
      }
    };
    uint4 v[QC];
    for (int m = grp; grp < ngr && m < p.M; m += ngr) {
      float amax = 0.0f;
      for (int c0 = 0; c0 < nch; c0 += QC * Tr) {
        load_round(m, c0, v);
#pragma unroll
        for (int i = 0; i < QC; ++i) amax = f16 ? chunk_absmax<W4_F16>(amax, v[i]) : chunk_absmax<W4_BF16>(amax, v[i]);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
      if (lane == 0) atomicMax(&qa_max[m], __float_as_uint(amax));   // amax >= 0: integer order
    }
    __syncthreads();
    for (int m = grp; grp < ngr && m < p.M; m += ngr) {
      const float s = __uint_as_float(qa_max[m]) / qmax;
      const float y = 1.0f / s;
      if (tr == 0) {
        qa_s[m] = s;
        if (blockIdx.x == 0 && p.a_scales_out) p.a_scales_out[m] = s;
      }
      for (int c0 = 0; c0 < nch; c0 += QC * Tr) {
        if (!keep) load_round(m, c0, v);
#pragma unroll
        for (int i = 0; i < QC; ++i) {
          const int c = c0 + tr + i * Tr;
          uint2 q = make_uint2(0u, 0u);
          if (s != 0.0f) {
            if (s >= 0x1p-100f)
              q = f16 ? quant_chunk<W4_F16, QT, true>(v[i], s, y) : quant_chunk<W4_BF16, QT, true>(v[i], s, y);
            else
              q = f16 ? quant_chunk<W4_F16, QT, false>(v[i], s, y) : quant_chunk<W4_BF16, QT, false>(v[i], s, y);
          }
          if (c < nch) *reinterpret_cast<uint2*>(qcodes + (uint32_t)(m * p.K + c * 8)) = q;
        }
      }
    }
    __syncthreads();
  };

  auto load_batch = [&](int buf, int kb) {   // kb: this wave's batch index in blocks of S
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = wave + (kb + u) * S;     // K block
      const bool in = k < KB && wave < S;    // waves past S only finalise
#pragma unroll
      for (int j = 0; j < NS; ++j)
        wv[buf][u][j] = __builtin_amdgcn_raw_buffer_load_b128(
            rw, (int)(in ? (uint32_t)((j * KB + k) * 1024) + w_lane : kOutOfRange), 0, W4_SKINNY_WPOLICY);
      if constexpr (kDma) {
        // rows past M and blocks past K read zeros (no traffic)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          buffer_load_lds16(ra, stage_of(buf, u) + h * 1024, in ? dma_off[h] + (uint32_t)(k * 128) : kOutOfRange);
      } else {
#pragma unroll
        for (int a = 0; a < AV; ++a) {
          if constexpr (QA)
            av[buf][u][a] = *reinterpret_cast<const u32x4*>(
                qcodes + (in && r < p.M ? a_lane + (uint32_t)(k * 128 + 16 * a) : qpad));
          else
            av[buf][u][a] = buffer_load16(ra, in ? a_lane + (uint32_t)(k * 128 * EB + 16 * a) : kOutOfRange);
        }
      }
    }
  };
  // loads a batch issues (a wait count for the batch issued before it)
  constexpr int kBatchLoads = U * (NS + (kDma ? 2 : AV));
  auto compute_batch = [&](int buf, int kb, bool pin, int after) {
    if constexpr (kDma) {
      // this batch's staged rows: its loads done (at most the next batch's
      // still in flight), then the fragment reads
      asm volatile("" ::: "memory");
      if (after) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kBatchLoads));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int a = 0; a < AV; ++a) av[buf][u][a] = *reinterpret_cast<const u32x4*>(stage_of(buf, u) + frag_off[a]);
    }
    // pin: loads issued before this point stay before it, and the weight
    // words enter an asm statement here, so none of this batch's work moves
    // above the previous refill (which would make its wait cover that refill)
    if (pin) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NS; ++j) asm volatile("" : "+v"(wv[buf][u][j]));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = wave + (kb + u) * S;
      if constexpr (SG > 1) {
        // groups of 64 or 32: each sub-group's dot products come from MFMAs
        // on the weight words of its lanes only, and are folded at once
        const int sgl = lane_subgroup<SG>(kq);
        f32x4 os[SG];
#pragma unroll
        for (int sg = 0; sg < SG; ++sg) {
          os[sg] = f32x4{};
          if constexpr (OP == OP_BF16) ones_mma_masked(av[buf][u], sgl == sg, os[sg]);
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          f16x2 nz = {};
          if constexpr (OP == OP_F16) {
            // the zero-point of the group this lane's weights belong to
            const float z = k < KB ? tz[(j * p.G + k * SG + sgl) * 16 + r] : 8.0f;
            const _Float16 h = (_Float16)(-(1024.0f + z));
            nz = f16x2{h, h};
          }
          uint32_t e[16];
          expand_weights<OP, FLIP>(wv[buf][u][j], nz, e);
          const int64_t n_d = (nb0 + j) * 16 + 4 * kq;
#pragma unroll
          for (int sg = 0; sg < SG; ++sg) {
            uint32_t es[16];
            mask_words<16>(e, sgl == sg, es);
            Acc t = Acc{};
            block_mma<OP>(es, av[buf][u], t);
            if (k < KB) {
              const int g = k * SG + sg;
              const int slot = (j * p.G + g) * 16 + 4 * kq;
              const f32x4 sv = *reinterpret_cast<const f32x4*>(&tsc[slot]);
              f32x4 zc = {};
              if constexpr (OP == OP_BF16) zc = *reinterpret_cast<const f32x4*>(&tz[slot]);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float pv = partial_value<OP>(t, os[sg], zc[i], i);
                if (partials) {
                  if (in_window(p, r, n_d + i)) store_partial<OP>(p, g, r, n_d + i, pv, 0);
                } else {
                  tot[j][i] = fmaf(pv, sv[i], tot[j][i]);
                }
              }
            }
          }
        }
        continue;
      }
      const int g = GROUPED ? k : 0;
      if constexpr (OP == OP_BF16 || PZ) ones_mma_16<OP>(av[buf][u], ones);
      if constexpr (ZP) ones_mma_i8(av[buf][u], ones_i);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        f16x2 nz = {};
        if constexpr (OP == OP_F16) {
          // pre-scaled zero-points: the raw code (its zero term comes with the fold)
          const float z = PZ ? 0.0f : GROUPED ? (k < KB ? tz[(j * p.G + g) * 16 + r] : 8.0f) : zrow[j];
          const _Float16 h = (_Float16)(-(1024.0f + z));
          nz = f16x2{h, h};
        }
        uint32_t e[16];
        expand_weights<OP, FLIP>(wv[buf][u][j], nz, e);
        block_mma<OP>(e, av[buf][u], acc[j]);
      }
      if constexpr (GROUPED) {
        if (k < KB) {
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            const int64_t n_d = (nb0 + j) * 16 + 4 * kq;
            // the group's scales and (bf16) 128 + z terms of D rows 4 kq + i
            const int slot = (j * p.G + g) * 16 + 4 * kq;
            const f32x4 sv = *reinterpret_cast<const f32x4*>(&tsc[slot]);
            f32x4 zc = {};
            if constexpr (OP == OP_BF16 || ZP || PZ) zc = *reinterpret_cast<const f32x4*>(&tz[slot]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // asymmetric int8: 16 * sum(a (u - z)), exact
              int32_t ia = 0;
              if constexpr (OP == OP_I8) ia = ZP ? acc[j][i] - (int32_t)zc[i] * ones_i[i] : acc[j][i];
              // pre-scaled zero-points: sum(a c) here (zc holds zs, taken below)
              const float pv = ZP ? (float)ia * 0.0625f
                               : PZ ? fmaf(OP == OP_BF16 ? -128.0f : 0.0f, ones[i], acc[j][i])
                                    : partial_value<OP>(acc[j], ones, zc[i], i);
              if (partials) {
                if (in_window(p, r, n_d + i))
                  store_partial<OP>(p, g, r, n_d + i, pv, ZP ? ia >> 4 : int_partial<OP>(acc[j], i));
              } else {
                const float pf = (OP == OP_I8) ? (float)ia : pv;
                tot[j][i] = fmaf(pf, sv[i], tot[j][i]);
                if constexpr (PZ) tot[j][i] = fmaf(-zc[i], ones[i], tot[j][i]);
              }
            }
          }
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[j] = Acc{};
        ones = f32x4{};
        ones_i = i32x4{};
      }
    }
  };

  // Table staging (grouped problems; the first round of loads is issued
  // before the first two batches, so that waiting for it does not wait for
  // the batches): thread t takes row t mod 16 NS of the workgroup's rows and
  // groups t / (16 NS) + i step, i < 8, so consecutive threads write
  // consecutive table words.  The stores are branch-free (a branch around a
  // store would make the compiler's wait for its load cover the batches
  // issued after it): groups past the last go to the table's pad.
  const int G = p.G;
  const int tab_total = kTab ? NS * 16 * G : 0;
  constexpr int RW = 16 * NS;
  const int srow = (int)threadIdx.x % RW;
  const int gstep = (int)blockDim.x / RW;   // blockDim.x is a multiple of 64
  const int gfirst = (int)threadIdx.x / RW;
  uint32_t tws[8], twz[8];
  auto stage_load = [&](int g0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int g = g0 + gfirst + t * gstep;
      const uint32_t idx = (uint32_t)((nb0 * 16 + srow) * G + g);
      if constexpr (GROUPED) tws[t] = load_word(rs, p.s_dtype, idx, g < G && !partials);
      if constexpr (OP == OP_BF16 || OP == OP_F16 || ZP) twz[t] = load_word(rz, zdt, idx, g < G && p.z);
    }
  };
  auto stage_store = [&](int g0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int g = g0 + gfirst + t * gstep;
      const uint32_t idx = (uint32_t)((nb0 * 16 + srow) * G + g);
      const int slot = g < G ? ((srow >> 4) * G + g) * 16 + (srow & 15) : tab_total + (srow & 15);
      if constexpr (GROUPED) {
        float sv = word_to_f32(tws[t], p.s_dtype, idx);
        if constexpr (OP == OP_I8) sv *= 0.0625f;   // the operand holds 16 w
        tsc[slot] = sv;
      }
      if constexpr (PZ)
        tz[slot] = word_to_f32(twz[t], zdt, idx);   // zs, the pre-scaled zero term
      else if constexpr (OP == OP_BF16)
        tz[slot] = 128.0f + (p.z ? word_to_f32(twz[t], zdt, idx) : 8.0f);
      else if constexpr (OP == OP_F16)
        tz[slot] = p.z ? word_to_f32(twz[t], zdt, idx) : 8.0f;
      if constexpr (ZP) tz[slot] = (p.z ? word_to_f32(twz[t], zdt, idx) : 8.0f) - 8.0f;
    }
  };
  // fused quantisation: the codes are in LDS before any batch is issued
  // (issuing the first batches' weights before the quantisation measured
  // slower: the quantisation's loads then wait for them)
  if constexpr (QA) quantise_rows();
  if constexpr (kTab) {
    stage_load(0);
    asm volatile("" ::: "memory");
    load_batch(0, 0);
    load_batch(1, U);
    asm volatile("" ::: "memory");
    stage_store(0);
    for (int g0 = 8 * gstep; g0 < G; g0 += 8 * gstep) {
      stage_load(g0);
      stage_store(g0);
    }
    // LDS writes done and visible; the two batches stay in flight
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // Both buffers are in flight: each step computes a buffer and refills it
    // with the batch two ahead (past K: zeros, no traffic).
    if (wave < S) {
      const int nbatch = (KB - wave + S - 1) / S;   // K blocks of this wave
      int kb = 0;
      for (; kb + 2 * U < nbatch; kb += 2 * U) {
        compute_batch(0, kb, true, 1);
        load_batch(0, kb + 2 * U);
        compute_batch(1, kb + U, true, 1);
        load_batch(1, kb + 3 * U);
      }
      compute_batch(0, kb, true, 1);
      compute_batch(1, kb + U, true, 0);
    }
  } else {
    // Each step issues the next batch, then computes the current one.
    if (wave < S) {
      const int nbatch = (KB - wave + S - 1) / S;   // K blocks of this wave
      load_batch(0, 0);
      int kb = 0;
      for (; kb + 2 * U < nbatch; kb += 2 * U) {
        load_batch(1, kb + U);
        compute_batch(0, kb, false, 1);
        load_batch(0, kb + 2 * U);
        compute_batch(1, kb + U, false, 1);
      }
      load_batch(1, kb + U);
      compute_batch(0, kb, false, 1);
      compute_batch(1, kb + U, false, 0);
    }
  }
  // (either way: whole pairs of batches, then the last pair, whose second
  // batch may lie past K; a loop without an exit in its middle keeps the next
  // batch's loads in flight across the back edge)

  // Sum the waves' results in wave order through LDS.
  __shared__ uint32_t red[skinny_max_waves(OP, GROUPED)][NS][64][4];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int64_t n_d = (nb0 + j) * 16 + 4 * kq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t bits;
      if constexpr (GROUPED) {
        bits = __float_as_uint(tot[j][i]);
      } else if constexpr (ZP) {
        const int32_t zc = (int32_t)(p.z ? word_to_f32(zpc[j][i], zdt, (uint32_t)(n_d + i) * p.G) : 8.0f) - 8;
        bits = (uint32_t)(acc[j][i] - zc * ones_i[i]);
      } else if constexpr (OP == OP_I8) {
        bits = (uint32_t)acc[j][i];
      } else {
        float zc = 0.0f;
        if constexpr (OP == OP_BF16)
          zc = 128.0f + (p.z ? word_to_f32(zpc[j][i], zdt, (uint32_t)(n_d + i) * p.G) : 8.0f);
        bits = __float_as_uint(partial_value<OP>(acc[j], ones, zc, i));
      }
      red[wave][j][lane][i] = bits;
    }
  }
  __syncthreads();
  if (GROUPED && partials) return;
  // One output element per thread (the launch provides at least 256 NS).
  if (ep_in) {
    const int j = ep_j, l = ep_l, i = ep_i;
    float fv = 0.0f;
    int32_t iv = 0;
    for (int w = 0; w < S; ++w) {
      if (!GROUPED && OP == OP_I8)
        iv += (int32_t)red[w][j][l][i];
      else
        fv += __uint_as_float(red[w][j][l][i]);
    }
    if (partials) {
      if (in_window(p, ep_m, ep_n)) store_partial<OP>(p, 0, ep_m, ep_n, fv, iv >> 4);
    } else {
      float v;
      if constexpr (GROUPED) {
        v = fv;
      } else {
        const float sn = word_to_f32(ep_s, p.s_dtype, (uint32_t)ep_n);
        v = (OP == OP_I8) ? (float)iv * (sn * 0.0625f) : fv * sn;
      }
      if constexpr (QA)
        v *= qa_s[ep_m];
      else if (p.a_scales)
        v *= __uint_as_float(ep_a);
      if (p.bias) v += word_to_f32(ep_b, p.out_dtype, (uint32_t)ep_n);
      store_out(p, ep_m, ep_n, v);
    }
  }
}

// ===========================================================================
// Tiled kernel.
//
// Workgroup = 4 waves; tile BM (rows of A) x BN = 4*NT*16 (columns of W);
// K steps of 128 (one PB-v1 block, one group).  Per step each wave expands
// its NT weight blocks once and multiplies them with the MT activation
// fragments of the step, read from LDS one m-tile ahead of use.
//
// Software pipeline (2 phases, ping-pong):
//   phase p computes step kb from LDS buffer p with weight registers wp, while
//   the global loads of step kb+1 (activation tile -> registers, weights ->
//   w(1-p)) are in flight; then the activation tile goes to LDS buffer 1-p and
//   one barrier separates the phases.  All global loads are buffer loads:
//   rows past M and blocks past N read as zero, and loads past the K range use
//   an out-of-range offset, so the loop has no divergent branches and the
//   compiler can count the outstanding loads exactly.
// ===========================================================================

// Workgroups per CU the tiled kernel is compiled for: three for the grouped
// 8-bit fold on 128-row tiles (its per-group VALU work overlaps the MFMAs of
// the other waves on the SIMD), two otherwise.
template <int OP, bool GROUPED, int MT, bool PARTIALS, bool ZP>
constexpr int tiled_min_blocks() {
  return (OP == OP_I8 || OP == OP_FP8) && GROUPED && !PARTIALS && !ZP && MT == 8 ? W4_TILED_FOLD_BLOCKS : 2;
}

template <int OP, bool GROUPED, bool FLIP, int NT, int MT, bool SPLIT, bool PARTIALS, bool ZP, int SG,
          bool PZ = false>
__global__ __launch_bounds__(256, (tiled_min_blocks<OP, GROUPED, MT, PARTIALS, ZP>())) void w4_gemm_tiled(GemmArgs p, int splitk) {
  using Acc = typename OpTraits<OP>::Acc;
  constexpr int EB = OpTraits<OP>::kElemBytes;
  constexpr int AV = act_vecs<OP>();
  constexpr int BM = MT * 16;
  constexpr int ROWB = 128 * EB;            // bytes of one activation row per K step
  constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  constexpr int RPL = 1024 / ROWB;          // rows filled by one wave-wide 16-byte load
  constexpr int LPT = BM / (4 * RPL);       // such loads per wave per tile
  constexpr int STAGE = BM * ROWB;          // bytes of one tile
  static_assert(BM % (4 * RPL) == 0, "tile rows must split evenly over the 4 waves");
  static_assert(3 * STAGE <= 65536, "fragment offsets must fit the LDS immediate");
  // Grouped problems also keep a two-slot table of column scales (and, bf16
  // W4A16, of 128 + z) after the three tile stages.  One LDS array holds
  // everything: a second array would give LDS accesses alias scopes, and the
  // compiler would then order the fragment reads after the in-flight tile
  // loads of later stages.
  constexpr bool kFold = GROUPED && !PARTIALS;
  constexpr int BNW = 4 * NT * 16;   // columns of the workgroup
  constexpr int kTables = kFold ? ((OP == OP_BF16 || ZP || PZ) ? 2 : 1) : 0;
  static_assert(!PZ || ((OP == OP_F16 || OP == OP_BF16) && GROUPED && !PARTIALS && SG == 1),
                "pre-scaled zero-points: grouped W4A16 outputs only");
  static_assert(!ZP || (OP == OP_I8 && FLIP), "zero-points: int8 operand from raw uint4 codes");
  static_assert(SG == 1 || (GROUPED && (OP == OP_F16 || OP == OP_BF16)), "sub-groups: grouped W4A16 only");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * STAGE + kTables * 2 * SG * BNW * 4];
  float* const gsc = reinterpret_cast<float*>(lds + 3 * STAGE);   // [2][SG][BNW]
  float* const gzc = gsc + 2 * SG * BNW;                          // [2][SG][BNW]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: scalar registers
  const int r = lane & 15;
  const int kq = lane >> 4;
  int bx, by, bz;
  tile_of_block(bx, by, bz);
  const int64_t m_base = (int64_t)bx * BM;
  const int64_t NB = p.N >> 4;
  const int64_t nb_base = (int64_t)by * (4 * NT) + wave * NT;
  const int KB = (int)(p.K >> 7);
  const int kb0 = (int)((int64_t)KB * bz / splitk);
  const int kb1 = (int)((int64_t)KB * (bz + 1) / splitk);
  constexpr bool partials = PARTIALS;  // verification mode: store group partials

  // Activation tile rows [m_base, m_base + BM): rows past M are out of range.
  const int64_t rows_valid = p.M - m_base < BM ? p.M - m_base : BM;
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(static_cast<const uint8_t*>(p.a) + m_base * p.K * EB, rows_valid * p.K * EB);
  // This wave's weight strips: NT n-blocks from nb_base, all K blocks.
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(reinterpret_cast<const uint8_t*>(p.b) + nb_base * KB * 1024, (NB - nb_base) * KB * 1024);
  const int sbytes = p.s_dtype == W4_F32 ? 4 : 2;
  // scales are absent (null) in the partials entry points: an empty buffer
  // (a product, not a branch: a branch here would wait for the kernel
  // arguments before anything else is issued)
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.s, (int64_t)(p.s != nullptr) * p.N * p.G * sbytes);
  const int zdt = p.z_dtype;    // zero-point storage dtype
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(p.z, p.z ? p.N * p.G * (zdt == W4_F32 ? 4 : 2) : 0);

  // Load j of this wave fills tile rows [(4 j + wave) RPL, +RPL); lane l
  // writes LDS bytes [16 l, 16 l + 16) of that range, i.e. row l / CPR, slot
  // l % CPR, which holds global chunk (l % CPR) ^ swz(row).
  uint32_t a_off[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int row = (4 * j + wave) * RPL + lane / CPR;
    const int chunk = (lane % CPR) ^ lds_swizzle<EB>(row);
    a_off[j] = (uint32_t)(row * p.K * EB + chunk * 16);
  }
  // Tile of step kb into LDS stage st.  Steps past the range read zeros.
  auto load_a = [&](int kb, int st) {
    const uint32_t base = kb < kb1 ? (uint32_t)(kb * ROWB) : kOutOfRange;
#pragma unroll
    for (int j = 0; j < LPT; ++j)
      buffer_load_lds16(ra, lds + st * STAGE + (4 * j + wave) * RPL * ROWB, base + a_off[j]);
  };
  auto load_w = [&](int kb, u32x4* w) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t off = kb < kb1 ? (uint32_t)(((nt * KB) + kb) * 1024 + lane * 16) : kOutOfRange;
      w[nt] = buffer_load16(rw, off);
    }
  };
  // Per-step side inputs, loaded one step ahead: group scales and (bf16)
  // zero-points of the D rows this lane owns, and (fp16 W4A16) the
  // zero-point of the operand row it feeds.
  struct Aux {
    uint32_t sc[NT][4];
    uint32_t zd[NT][4];
    uint32_t wz[NT];
  };
  auto load_aux = [&](int kb, Aux& x) {
    if constexpr (GROUPED) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (PARTIALS && (OP == OP_BF16 || ZP)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t n = (uint32_t)((nb_base + nt) * 16 + 4 * kq + i);
            x.zd[nt][i] = load_word(rz, zdt, n * p.G + kb, kb < kb1 && p.z);
          }
        }
        if constexpr (OP == OP_F16 && !PZ)
          x.wz[nt] = load_word(rz, zdt, (uint32_t)(((nb_base + nt) * 16 + r) * p.G + kb * SG + lane_subgroup<SG>(kq)),
                               kb < kb1 && p.z);
      }
    }
  };
  // fp16 W4A16 per channel: one zero-point per operand row for all of K
  // (through the zero-point buffer: rows past N, in the last column tile,
  // read nothing).
  f16x2 nz_fixed[NT];
  if constexpr (OP == OP_F16 && !GROUPED) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t n = (nb_base + nt) * 16 + r;
      const uint32_t zi = (uint32_t)n * (uint32_t)p.G;
      const float z = p.z ? word_to_f32(load_word(rz, zdt, zi, n < p.N), zdt, zi) : 8.0f;
      const _Float16 h = (_Float16)(-(1024.0f + z));
      nz_fixed[nt] = f16x2{h, h};
    }
  }

  Acc acc[NT][MT];
  f32x4 tot[NT][MT];
  f32x4 ones[MT];
  i32x4 onesi[MT];   // asymmetric int8: 16 * sum(a) of the tile rows
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[nt][mt] = Acc{};
      tot[nt][mt] = f32x4{};
    }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ones[mt] = f32x4{};
    onesi[mt] = i32x4{};
  }

  // LDS offset of this lane's fragment chunk j in rows r (+ 16 mt).
  int frag_off[AV];
#pragma unroll
  for (int j = 0; j < AV; ++j) frag_off[j] = r * ROWB + (((kq * AV + j) ^ lds_swizzle<EB>(r)) * 16);

  // Grouped problems fold each group's dot products into fp32 totals with the
  // group scale.  The scales (and bf16 zero-point terms 128 + z) of the
  // workgroup's BN columns are converted once per column and step by one
  // thread each into the two-slot LDS table (slot (kb - kb0) & 1), written
  // one step ahead; a lane then reads its four rows' values with one 16-byte
  // LDS read per n-block.  int8 scales carry the 1/16 of the 16 w operand.
  const int col = tid % BNW;
  const uint32_t col_n = (uint32_t)((int64_t)by * BNW + col);
  // raw words of the column for the step being prefetched (SG groups per step)
  uint32_t col_sw[SG], col_zw[SG];
#pragma unroll
  for (int sg = 0; sg < SG; ++sg) col_sw[sg] = col_zw[sg] = 0;
  auto load_col = [&](int kb) {
    if constexpr (kFold) {
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        const uint32_t idx = col_n * (uint32_t)p.G + (uint32_t)(kb * SG + sg);
        col_sw[sg] = load_word(rs, p.s_dtype, idx, kb < kb1 && col_n < (uint32_t)p.N);
        if constexpr (OP == OP_BF16 || ZP || PZ)
          col_zw[sg] = load_word(rz, zdt, idx, kb < kb1 && p.z && col_n < (uint32_t)p.N);
      }
    }
  };
  auto store_col = [&](int kb) {
    if constexpr (kFold) {
      const int slot = (kb - kb0) & 1;
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        const uint32_t idx = col_n * (uint32_t)p.G + (uint32_t)(kb * SG + sg);
        const int at = (slot * SG + sg) * BNW + col;
        float sv = word_to_f32(col_sw[sg], p.s_dtype, idx);
        if constexpr (OP == OP_I8) sv *= 0.0625f;
        gsc[at] = sv;
        if constexpr (PZ)
          gzc[at] = word_to_f32(col_zw[sg], zdt, idx);   // zs, the pre-scaled zero term
        else if constexpr (OP == OP_BF16)
          gzc[at] = 128.0f + (p.z ? word_to_f32(col_zw[sg], zdt, idx) : 8.0f);
        if constexpr (ZP) gzc[at] = (p.z ? word_to_f32(col_zw[sg], zdt, idx) : 8.0f) - 8.0f;
      }
    }
  };

  // One K step: expand this step's weights, refill their registers with the
  // weights of step kb + 2, then run the MFMAs on LDS stage st.
  auto step = [&](int kb, int st, u32x4* w, const Aux& x) {
    // The weight words enter an asm statement that follows the barrier, so
    // their expansion (and the wait for their loads) stays in this step
    // instead of being hoisted into the previous one.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(w[nt]));
    uint32_t e[NT][16];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f16x2 nz = {};
      if constexpr (OP == OP_F16) {
        if constexpr (PZ) {
          const _Float16 h = (_Float16)(-1024.0f);   // the raw code; the zero term comes with the fold
          nz = f16x2{h, h};
        } else if constexpr (GROUPED) {
          const uint32_t zi = (uint32_t)(((nb_base + nt) * 16 + r) * p.G + kb * SG + lane_subgroup<SG>(kq));
          const _Float16 h = (_Float16)(-(1024.0f + (p.z ? word_to_f32(x.wz[nt], zdt, zi) : 8.0f)));
          nz = f16x2{h, h};
        } else {
          nz = nz_fixed[nt];
        }
      }
      expand_weights<OP, FLIP>(w[nt], nz, e[nt]);
    }
    // Every expanded word exists before the weight registers are refilled:
    // the old words die here, so the refill reuses their registers and no
    // copy (and no wait for the refill) is needed at the loop's back edge.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pin_words<kExpandedWords<OP>>(e[nt]);
    load_w(kb + 2, w);
    asm volatile("" ::: "memory");  // issue the refill before the LDS reads
    const uint8_t* src = lds + st * STAGE;
    u32x4 af[MT][AV];
    auto load_frag = [&](int mt) {
#pragma unroll
      for (int j = 0; j < AV; ++j)
        af[mt][j] = *reinterpret_cast<const u32x4*>(src + mt * 16 * ROWB + frag_off[j]);
    };
    // The grouped fold's steps are fenced region by region, so its fragment
    // reads are issued in its loop, two tile rows ahead (three rows live);
    // the other paths read them all here and order them with the MFMAs.
    constexpr bool kFoldFrag = kFold && SG == 1;
#pragma unroll
    for (int mt = 0; mt < (kFoldFrag ? (MT < 2 ? MT : 2) : MT); ++mt) load_frag(mt);
    if constexpr (SG > 1) {
      // groups of 64 or 32: per sub-group, MFMAs on the weight words of its
      // lanes only, folded (or stored) at once
      const int sgl = lane_subgroup<SG>(kq);
      const int slot = (kb - kb0) & 1;
      // sub-group outermost: only its masked weight words are live
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        const int g = kb * SG + sg;
        uint32_t es[NT][16];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          mask_words<16>(e[nt], sgl == sg, es[nt]);
          pin_words<16>(es[nt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 os = {};
          if constexpr (OP == OP_BF16) ones_mma_masked(af[mt], sgl == sg, os);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int64_t n_d = (nb_base + nt) * 16 + 4 * kq;
            Acc t = Acc{};
            block_mma<OP>(es[nt], af[mt], t);
            if constexpr (PARTIALS) {
              const int64_t m = m_base + mt * 16 + r;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                if (m < p.M && n_d < p.N && in_window(p, m, n_d + i)) {
                  const float zc = (OP == OP_BF16) ? 128.0f + zero_point(p, n_d + i, g) : 0.0f;
                  store_partial<OP>(p, g, m, n_d + i, partial_value<OP>(t, os, zc, i), 0);
                }
              }
            } else {
              const int at = (slot * SG + sg) * BNW + (wave * NT + nt) * 16 + 4 * kq;
              const f32x4 sv = *reinterpret_cast<const f32x4*>(&gsc[at]);
              f32x4 zc = {};
              if constexpr (OP == OP_BF16) zc = *reinterpret_cast<const f32x4*>(&gzc[at]);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                tot[nt][mt][i] = fmaf(partial_value<OP>(t, os, zc[i], i), sv[i], tot[nt][mt][i]);
            }
          }
        }
      }
    } else if constexpr (kFold) {
      // This group's scales (and bf16 128 + z terms) for the lane's D rows.
      const int slot = (kb - kb0) & 1;
      f32x4 scv[NT], zcv[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        scv[nt] = *reinterpret_cast<const f32x4*>(&gsc[slot * BNW + (wave * NT + nt) * 16 + 4 * kq]);
        if constexpr (OP == OP_BF16 || ZP || PZ)
          zcv[nt] = *reinterpret_cast<const f32x4*>(&gzc[slot * BNW + (wave * NT + nt) * 16 + 4 * kq]);
      }
      // Row mt's MFMAs start from zero; row mt - 1 is folded while they run.
      auto fold_block = [&](int nt, int mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float pv;
          if constexpr (ZP)
            pv = (float)(acc[nt][mt][i] - (int32_t)zcv[nt][i] * onesi[mt][i]);
          else if constexpr (OP == OP_I8)
            pv = (float)acc[nt][mt][i];
          else if constexpr (PZ)
            pv = fmaf(OP == OP_BF16 ? -128.0f : 0.0f, ones[mt][i], acc[nt][mt][i]);
          else if constexpr (OP == OP_BF16)
            pv = fmaf(-zcv[nt][i], ones[mt][i], acc[nt][mt][i]);
          else
            pv = acc[nt][mt][i];
          tot[nt][mt][i] = fmaf(pv, scv[nt][i], tot[nt][mt][i]);
          if constexpr (PZ) tot[nt][mt][i] = fmaf(-zcv[nt][i], ones[mt][i], tot[nt][mt][i]);
        }
      };
      // Issue order, pinned: per tile row, the fragment reads of row mt + 2,
      // then per n-block the row's MFMAs followed by the fold of the same
      // n-block of row mt - 1 (whose MFMAs finished a row earlier), so the
      // fold's VALU work runs in the MFMAs' shadow.
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt + 2 < MT) load_frag(mt + 2);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          Acc t = Acc{};
          block_mma<OP>(e[nt], af[mt], t);
          acc[nt][mt] = t;
          if (nt == NT - 1 && (OP == OP_BF16 || PZ)) {
            f32x4 o = f32x4{};
            ones_mma_16<OP>(af[mt], o);
            ones[mt] = o;
          }
          if (nt == NT - 1 && ZP) {
            i32x4 o = i32x4{};
            ones_mma_i8(af[mt], o);
            onesi[mt] = o;
          }
          if (mt > 0) fold_block(nt, mt - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) fold_block(nt, MT - 1);
    } else {
      // 64-row int8 tiles: the step's MFMAs form a region of their own.
      // Otherwise the scheduler moves about a third of them past the next
      // step's barrier, which measured 3-5% slower at M = 512-1024.  The
      // 128-row tile is left alone: split there, it runs out of registers.
      constexpr bool kFence = MT == 4 && OP == OP_I8;
      if constexpr (kFence) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) block_mma<OP>(e[nt], af[mt], acc[nt][mt]);
        if constexpr (OP == OP_BF16) ones_mma(af[mt], ones[mt]);
        if constexpr (ZP) ones_mma_i8(af[mt], onesi[mt]);
      }
      // Issue order: the fragment reads of tile row mt + 2 go out with the
      // MFMAs of row mt, so each read has two rows of MFMAs to land.
      constexpr int kMfmaPerRow = NT * kMfmaPerBlock<OP> + (OP == OP_BF16 ? 4 : 0) + (ZP ? 2 : 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * AV, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPerRow, 0);
        if (mt + 2 < MT) __builtin_amdgcn_sched_group_barrier(0x100, AV, 0);
      }
      if constexpr (kFence) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (GROUPED && PARTIALS && SG == 1) {
      // verification mode: store each group's dot products
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int64_t n_d = (nb_base + nt) * 16 + 4 * kq;
        float zc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t idx = (uint32_t)(n_d + i) * p.G + kb;
          const float z = p.z ? word_to_f32(x.zd[nt][i], zdt, idx) : 8.0f;
          zc[i] = (OP == OP_BF16) ? 128.0f + z : (ZP ? z - 8.0f : 0.0f);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int64_t m = m_base + mt * 16 + r;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            int32_t ia = 0;
            if constexpr (ZP) ia = acc[nt][mt][i] - (int32_t)zc[i] * onesi[mt][i];
            const float pv = ZP ? (float)ia * 0.0625f : partial_value<OP>(acc[nt][mt], ones[mt], zc[i], i);
            if (m < p.M && n_d < p.N && in_window(p, m, n_d + i))
              store_partial<OP>(p, kb, m, n_d + i, pv, ZP ? ia >> 4 : int_partial<OP>(acc[nt][mt], i));
          }
          acc[nt][mt] = Acc{};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        ones[mt] = f32x4{};
        onesi[mt] = i32x4{};
      }
    }
  };

  // Pipeline: step kb computes from LDS stage kb mod 3 while the tiles of
  // steps kb + 1 and kb + 2 are in flight, and from weight registers that are
  // refilled with step kb + 2 as soon as they are expanded.  Each step issues
  // its side inputs (column scales two steps ahead, per-lane values one step
  // ahead), then LPT tile loads, then NT weight loads, so at a barrier at most
  // LPT + NT operations issued after the tile the next step reads (those of
  // the previous step) may still be outstanding.
  constexpr int kAfterTile = LPT + NT;
  u32x4 w0[NT], w1[NT];
  Aux x0, x1;
  // The prologue issues in the loop's order (the compiler's waits at the
  // loop head must hold for the first entry as well).
  load_col(kb0);
  store_col(kb0);
  load_col(kb0 + 1);
  load_aux(kb0, x0);
  asm volatile("" ::: "memory");
  load_a(kb0, 0);
  load_w(kb0, w0);
  asm volatile("" ::: "memory");
  load_a(kb0 + 1, 1);
  load_w(kb0 + 1, w1);
  asm volatile("" ::: "memory");
  // Whole pairs of steps, then an odd last step: a loop without an exit in
  // its middle, so the compiler's wait analysis sees only the real order.
  auto phase = [&](int kb, int st, u32x4* w, Aux& cur, Aux& next) {
    stage_barrier<kAfterTile>();
    store_col(kb + 1);
    load_col(kb + 2);
    load_aux(kb + 1, next);
    load_a(kb + 2, st == 0 ? 2 : st - 1);
    step(kb, st, w, cur);
  };
  int st = 0;
  int kb = kb0;
  for (int pairs = (kb1 - kb0) >> 1; pairs > 0; --pairs, kb += 2) {
    phase(kb, st, w0, x0, x1);
    st = st == 2 ? 0 : st + 1;
    phase(kb + 1, st, w1, x1, x0);
    st = st == 2 ? 0 : st + 1;
  }
  if ((kb1 - kb0) & 1) phase(kb, st, w0, x0, x1);
  // Drain the loads issued past the last step before the workgroup's LDS is
  // released.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  if (GROUPED && partials) return;
  // Epilogue: lane holds rows n_d..n_d+3 of column m for every (nt, mt).
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t n_d = (nb_base + nt) * 16 + 4 * kq;
    if (n_d >= p.N) continue;
    float zc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (OP == OP_BF16 && !GROUPED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) zc[i] = 128.0f + zero_point(p, n_d + i, 0);
    }
    if constexpr (ZP && !GROUPED) {
#pragma unroll
      for (int i = 0; i < 4; ++i) zc[i] = zero_point(p, n_d + i, 0) - 8.0f;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = m_base + mt * 16 + r;
      if (m >= p.M) continue;
      uint32_t bits[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (GROUPED)
          bits[i] = __float_as_uint(tot[nt][mt][i]);
        else if constexpr (ZP)
          bits[i] = (uint32_t)(acc[nt][mt][i] - (int32_t)zc[i] * onesi[mt][i]);
        else if constexpr (OP == OP_I8)
          bits[i] = (uint32_t)acc[nt][mt][i];
        else
          bits[i] = __float_as_uint(partial_value<OP>(acc[nt][mt], ones[mt], zc[i], i));
      }
      if constexpr (SPLIT) {
        uint32_t* slot = static_cast<uint32_t*>(p.ws) + ((int64_t)bz * p.M + m) * p.N + n_d;
        *reinterpret_cast<u32x4*>(slot) = u32x4{bits[0], bits[1], bits[2], bits[3]};
      } else if (partials) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (in_window(p, m, n_d + i))
            store_partial<OP>(p, 0, m, n_d + i, __uint_as_float(bits[i]), (int32_t)bits[i] >> 4);
      } else {
        uint16_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = finalize<OP, GROUPED>(p, m, n_d + i, __uint_as_float(bits[i]), (int32_t)bits[i]);
          o[i] = p.out_dtype == W4_F16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
        }
        uint2 packed = make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + m * p.N + n_d) = packed;
      }
    }
  }
}

// Four consecutive elements [i, i + 4) of an fp32 / fp16 / bf16 array as fp32
// (i a multiple of 4; the array 16-byte aligned).
__device__ __forceinline__ f32x4 load_quad_f32(const void* p, int dtype, int64_t i) {
  if (dtype == W4_F32) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    return f32x4{v.x, v.y, v.z, v.w};
  }
  const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
  const uint32_t h[4] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16};
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = dtype == W4_F16 ? f16_bits_to_f32(h[j]) : bf16_bits_to_f32(h[j]);
  return r;
}

// Sum the split-K slots of the tiled kernel in split order, then the epilogue.
// A thread owns four consecutive columns of one row.  Its epilogue operands
// (per-channel scales, bias, the row's activation scale) are loaded first, so
// that they are in flight with the slots; the slots are loaded eight at a
// time (all in flight together; slots past the last read zero) and added in
// slot order.  The epilogue is the one `finalize` computes, term for term.
template <int OP, bool GROUPED>
__global__ __launch_bounds__(256) void w4_splitk_reduce(GemmArgs p, int splitk) {
  const int64_t quads = p.N >> 2;
  const int64_t total = p.M * quads;
  const bool partials = p.mode == MODE_PARTIALS;
  const int64_t slot_words = p.M * p.N;
  // the workspace as a buffer: offsets are per slot, so any M * N * 4 below
  // the descriptor limit works; larger problems use plain loads
  const bool use_rsrc = slot_words * 4 * splitk < 0x7FFFFFF0LL;
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(p.ws, use_rsrc ? slot_words * 4 * splitk : 0);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = t / quads;
    const int64_t n = (t - m * quads) * 4;
    const int64_t base = m * p.N + n;   // word index in slot 0
    f32x4 sv{1.0f, 1.0f, 1.0f, 1.0f}, bv{0.0f, 0.0f, 0.0f, 0.0f};
    float am = 1.0f;
    if (!partials) {
      if (!GROUPED) sv = load_quad_f32(p.s, p.s_dtype, n);
      if (p.bias) bv = load_quad_f32(p.bias, p.out_dtype, n);
      if (p.a_scales) am = p.a_scales[m];
    }
    float fv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int32_t iv[4] = {0, 0, 0, 0};
    auto add = [&](const u32x4& v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!GROUPED && OP == OP_I8)
          iv[i] += (int32_t)v[i];
        else
          fv[i] += __uint_as_float(v[i]);
      }
    };
    if (use_rsrc) {
      for (int s0 = 0; s0 < splitk; s0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          v[q] = buffer_load16(rws, s0 + q < splitk ? (uint32_t)(((s0 + q) * slot_words + base) * 4) : kOutOfRange);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (s0 + q < splitk) add(v[q]);
      }
    } else {
      for (int s = 0; s < splitk; ++s)
        add(*reinterpret_cast<const u32x4*>(static_cast<const uint32_t*>(p.ws) + s * slot_words + base));
    }
    if (partials) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (in_window(p, m, n + i)) store_partial<OP>(p, 0, m, n + i, fv[i], iv[i] >> 4);
    } else {
      uint16_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v;
        if constexpr (GROUPED)
          v = fv[i];
        else
          v = (OP == OP_I8) ? (float)iv[i] * (sv[i] * 0.0625f) : fv[i] * sv[i];
        if (p.a_scales) v *= am;
        if (p.bias) v += bv[i];
        o[i] = p.out_dtype == W4_F16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
      }
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + m * p.N + n) =
          make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
    }
  }
}

// ===========================================================================
// Host-side launchers.
// ===========================================================================
hipError_t launch_splitk_reduce(const GemmArgs& args, int op, bool grouped, int splitk, hipStream_t stream) {
  const int64_t total = args.M * (args.N / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks), block(256);
  switch (op * 2 + (grouped ? 1 : 0)) {
    case OP_I8 * 2: hipLaunchKernelGGL((w4_splitk_reduce<OP_I8, false>), grid, block, 0, stream, args, splitk); break;
    case OP_I8 * 2 + 1: hipLaunchKernelGGL((w4_splitk_reduce<OP_I8, true>), grid, block, 0, stream, args, splitk); break;
    case OP_FP8 * 2: hipLaunchKernelGGL((w4_splitk_reduce<OP_FP8, false>), grid, block, 0, stream, args, splitk); break;
    case OP_FP8 * 2 + 1: hipLaunchKernelGGL((w4_splitk_reduce<OP_FP8, true>), grid, block, 0, stream, args, splitk); break;
    case OP_F16 * 2: hipLaunchKernelGGL((w4_splitk_reduce<OP_F16, false>), grid, block, 0, stream, args, splitk); break;
    case OP_F16 * 2 + 1: hipLaunchKernelGGL((w4_splitk_reduce<OP_F16, true>), grid, block, 0, stream, args, splitk); break;
    case OP_BF16 * 2: hipLaunchKernelGGL((w4_splitk_reduce<OP_BF16, false>), grid, block, 0, stream, args, splitk); break;
    case OP_BF16 * 2 + 1: hipLaunchKernelGGL((w4_splitk_reduce<OP_BF16, true>), grid, block, 0, stream, args, splitk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

void tiled_tile(int op, bool grouped, int tall, int* bm, int* bn, bool zp) {
  // 8-bit operands: 64 x 256, or the tall tile, 128 x 256 for int8 per
  // channel and 128 x 128 otherwise (2 n-blocks per wave: grouped, fp8 and
  // zero-point waves spend more VALU (or registers) per weight block, which 8
  // tile rows amortise)
  if (op == OP_I8 || op == OP_FP8) {
    const bool wide = op == OP_I8 && !grouped && !zp;
    *bm = tall ? 128 : 64;
    *bn = (tall && !wide) ? 128 : 256;
  } else {
    *bm = 64;
    *bn = 128;
  }
}

template <int OP, bool GROUPED, bool FLIP, bool ZP = false, int SG = 1, bool PZ = false>
static hipError_t launch_typed(const GemmArgs& args, const GemmPlan& plan, hipStream_t stream) {
  if (plan.path == PATH_SKINNY) {
    // S waves split K; at least 4 NS waves are launched so that every output
    // element of the workgroup has a thread in the epilogue.
    const int S = plan.splitk;
    const int ns = plan.bn / 16;
    const unsigned threads = 64u * (unsigned)(S > 4 * ns ? S : 4 * ns);
    const dim3 grid((unsigned)(args.N / plan.bn));
    const bool part = args.mode == MODE_PARTIALS;
    // tables (checked by the plan), then (staged 8-bit activations) each
    // wave's two staging buffers of U 2 KiB blocks
    constexpr bool kByteAct = OP == OP_I8 || OP == OP_FP8;
    const bool da = kByteAct && args.M >= 8;
    const int su = GROUPED ? (ns == 1 ? W4_SKINNY_UG1 : W4_SKINNY_UG2) : W4_SKINNY_U8;
    const size_t tab = (((size_t)skinny_table_bytes(OP, GROUPED, args.G, ns, ZP) + 15) & ~(size_t)15) +
                       (da ? (size_t)(threads / 64) * 2 * su * 2048 : 0);
    if (args.x) {
      // fused quantisation: the codes and their pad follow the tables
      if constexpr ((OP == OP_I8 || OP == OP_FP8) && !ZP && SG == 1) {
        const size_t lds = (size_t)skinny_table_bytes(OP, GROUPED, args.G, ns, ZP) + (size_t)(args.M * args.K) + 32;
        if (ns == 2)
          hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 2, false, false, 1, true>), grid, dim3(threads), lds,
                             stream, args, S);
        else
          hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 1, false, false, 1, true>), grid, dim3(threads), lds,
                             stream, args, S);
        return hipGetLastError();
      } else {
        return hipErrorInvalidValue;
      }
    }
    if constexpr (kByteAct) {
      if (da) {
        if (ns == 2) {
          if (part)
            hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 2, true, ZP, SG, false, false, true>), grid,
                               dim3(threads), tab, stream, args, S);
          else
            hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 2, false, ZP, SG, false, false, true>), grid,
                               dim3(threads), tab, stream, args, S);
        } else {
          if (part)
            hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 1, true, ZP, SG, false, false, true>), grid,
                               dim3(threads), tab, stream, args, S);
          else
            hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 1, false, ZP, SG, false, false, true>), grid,
                               dim3(threads), tab, stream, args, S);
        }
        return hipGetLastError();
      }
    }
    if (ns == 2) {
      if (part)
        hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 2, true, ZP, SG, false>), grid, dim3(threads), tab, stream, args, S);
      else
        hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 2, false, ZP, SG, false, PZ>), grid, dim3(threads), tab, stream, args, S);
    } else {
      if (part)
        hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 1, true, ZP, SG, false>), grid, dim3(threads), tab, stream, args, S);
      else
        hipLaunchKernelGGL((w4_gemm_skinny<OP, GROUPED, FLIP, 1, false, ZP, SG, false, PZ>), grid, dim3(threads), tab, stream, args, S);
    }
    return hipGetLastError();
  }
  if (args.x) return hipErrorInvalidValue;   // the fused quantisation exists in the small-M kernel only
  constexpr bool kByte = (OP == OP_I8 || OP == OP_FP8);
  auto finish = [&]() -> hipError_t {
    hipError_t e = hipGetLastError();
    // grouped partials are stored by the tiled kernel itself
    if (e != hipSuccess || plan.splitk == 1 || (GROUPED && args.mode == MODE_PARTIALS)) return e;
    return launch_splitk_reduce(args, OP, GROUPED, plan.splitk, stream);
  };
  auto launch = [&](auto mt_tag, auto nt_tag) {
    constexpr int MT = decltype(mt_tag)::value;
    constexpr int NT = decltype(nt_tag)::value;
    const int64_t BM = MT * 16, BN = NT * 64;
    const dim3 grid((unsigned)((args.M + BM - 1) / BM), (unsigned)((args.N + BN - 1) / BN),
                    (unsigned)plan.splitk);
    const bool part = args.mode == MODE_PARTIALS;
    if (plan.splitk > 1) {
      if (part)
        hipLaunchKernelGGL((w4_gemm_tiled<OP, GROUPED, FLIP, NT, MT, true, true, ZP, SG>), grid, dim3(256), 0, stream,
                           args, plan.splitk);
      else
        hipLaunchKernelGGL((w4_gemm_tiled<OP, GROUPED, FLIP, NT, MT, true, false, ZP, SG, PZ>), grid, dim3(256), 0, stream,
                           args, plan.splitk);
    } else {
      if (part)
        hipLaunchKernelGGL((w4_gemm_tiled<OP, GROUPED, FLIP, NT, MT, false, true, ZP, SG>), grid, dim3(256), 0, stream,
                           args, 1);
      else
        hipLaunchKernelGGL((w4_gemm_tiled<OP, GROUPED, FLIP, NT, MT, false, false, ZP, SG, PZ>), grid, dim3(256), 0, stream,
                           args, 1);
    }
  };
  if constexpr (kByte) {
    if (plan.bm == 128 && plan.bn == 256) {
      // the 128 x 256 tile exists for symmetric int8 per channel only
      if constexpr (OP == OP_I8 && !GROUPED && !ZP)
        launch(std::integral_constant<int, 8>{}, std::integral_constant<int, 4>{});
      else
        return hipErrorInvalidValue;
    } else if (plan.bm == 128)
      launch(std::integral_constant<int, 8>{}, std::integral_constant<int, 2>{});
    else if (plan.bn == 128)
      launch(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{});
    else
      launch(std::integral_constant<int, 4>{}, std::integral_constant<int, 4>{});
  } else if constexpr (SG == 4) {
    // groups of 32: four sub-group passes per block; 32-row tiles keep the
    // activation fragments and totals in registers
    launch(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
  } else {
    launch(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{});
  }
  return finish();
}

hipError_t launch_gemm(const GemmArgs& args, int op, bool grouped, bool flip, bool zp, const GemmPlan& plan,
                       hipStream_t stream) {
  if (plan.path == PATH_STREAM) return zp ? hipErrorInvalidValue : launch_stream(args, op, grouped, flip, plan, stream);
  if (plan.path == PATH_PINGPONG) {
    if (op != OP_I8 || grouped || zp || args.x || args.z) return hipErrorInvalidValue;
    return launch_pingpong(args, flip, plan, stream);
  }
  if (zp) {   // asymmetric int8 W4A8 (the API admits no other combination)
    if (op != OP_I8 || !flip) return hipErrorInvalidValue;
    return grouped ? launch_typed<OP_I8, true, true, true>(args, plan, stream)
                   : launch_typed<OP_I8, false, true, true>(args, plan, stream);
  }
#define W4_DISPATCH(OPV)                                                          \
  if (grouped)                                                                    \
    return flip ? launch_typed<OPV, true, true>(args, plan, stream)               \
                : launch_typed<OPV, true, false>(args, plan, stream);             \
  return flip ? launch_typed<OPV, false, true>(args, plan, stream)                \
              : launch_typed<OPV, false, false>(args, plan, stream);
  switch (op) {
    case OP_I8: W4_DISPATCH(OP_I8)
    case OP_FP8: W4_DISPATCH(OP_FP8)
    case OP_F16:
    default: {
      // W4A16 groups of 128, 64 or 32: 1, 2 or 4 groups per 128-deep block
      const int64_t sg = grouped ? 128 * (int64_t)args.G / args.K : 1;
      if (args.prescaled_zeros) {   // groups of 128 only (the API admits no other)
        if (!grouped || sg != 1 || args.mode != MODE_OUTPUT) return hipErrorInvalidValue;
        return op == OP_F16 ? launch_typed<OP_F16, true, false, false, 1, true>(args, plan, stream)
                            : launch_typed<OP_BF16, true, false, false, 1, true>(args, plan, stream);
      }
      if (op == OP_F16) {
        if (!grouped) return launch_typed<OP_F16, false, false>(args, plan, stream);
        return sg == 4 ? launch_typed<OP_F16, true, false, false, 4>(args, plan, stream)
               : sg == 2 ? launch_typed<OP_F16, true, false, false, 2>(args, plan, stream)
                         : launch_typed<OP_F16, true, false>(args, plan, stream);
      }
      if (!grouped) return launch_typed<OP_BF16, false, false>(args, plan, stream);
      return sg == 4 ? launch_typed<OP_BF16, true, false, false, 4>(args, plan, stream)
             : sg == 2 ? launch_typed<OP_BF16, true, false, false, 2>(args, plan, stream)
                       : launch_typed<OP_BF16, true, false>(args, plan, stream);
    }
  }
#undef W4_DISPATCH
}

}  // namespace w4
