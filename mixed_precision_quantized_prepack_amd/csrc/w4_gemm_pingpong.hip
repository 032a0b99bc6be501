// Ping-pong tiled GEMM kernel for gfx950: symmetric int8 W4A8 per channel at
// large M.
//
//   out[m,n] = RNE( s_a[m] * s[n] * sum_k a[m,k] * w[n,k] + bias[n] )
//
// ("support W4A8 Marlin kernel": per-channel W4A8 with per-token activation
// scales; its GEMM benchmark shape N = 8192, K = 21760.)
#include "w4_gemm_common.h"

namespace w4 {

// ===========================================================================
// One workgroup of eight waves per CU computes a 256 x 256 tile (KS false) or
// a 128 x 256 tile (KS true) as two groups of four waves, each the tiled
// kernel's 128 x 256 tile (wave w of a group owns 4 16-column n-blocks across
// its 128 rows; its own half of a three-stage LDS ring for the activation
// rows; weights in registers, two steps ahead).  Without KS the groups take
// rows 0-127 and 128-255; with KS both take the same rows and alternate K
// steps (group 0 the even steps of the range, group 1 the odd ones), and
// their exact int32 sums are added through LDS at the end.  A group
// alternates two phases per 128-deep K step:
//   V: wait for the step's loads, expand the weights, issue the loads of the
//      step two ahead;
//   M: the step's fragment reads and 64 MFMAs per wave.
// Phases are slots between workgroup barriers, and group 1 runs one slot
// behind group 0, so in each slot one group's MFMAs share every SIMD with the
// other group's expansion and loads.  (Two independent workgroups per CU, the
// tiled kernel's arrangement, drift into step and leave the MFMAs idle while
// both expand.)  The two groups share no LDS and no registers; the barriers
// only pace them.
// ===========================================================================
template <bool KS, bool FLIP, bool SPLIT, bool PARTIALS>
__global__ __launch_bounds__(512, 1) void w4_gemm_pingpong(GemmArgs p, int splitk) {
  constexpr int MT = 8;
  constexpr int OP = OP_I8;
  using Acc = typename OpTraits<OP>::Acc;
  constexpr int AV = act_vecs<OP>();
  constexpr int NT = 4;
  constexpr int GM = 16 * MT;               // rows of one group
  constexpr int ROWB = 128, CPR = 8, RPL = 8;
  constexpr int HALF = GM * ROWB;           // one group's rows of a stage
  constexpr int STAGE = 2 * HALF;
  constexpr int LPT = GM / (4 * RPL);        // tile loads per wave per step
  constexpr int kAfter = LPT + NT;           // loads issued after a step's own
  constexpr int STRIDE = KS ? 2 : 1;         // K steps between a group's steps
  constexpr int RED = 4 * NT * MT * 64 * 16; // the K-split halves' sum: group 1's accumulators
  constexpr int LDS = (KS && RED > 3 * STAGE) ? RED : 3 * STAGE;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int gw = wave & 3;
  const int r = lane & 15;
  const int kq = lane >> 4;
  int bx, by, bz;
  // 256 x 256 tiles: 32 resident per XCD as 4 m-tiles x 8 n-tiles (equal
  // activation and weight bytes per K step); 128 x 256 tiles as the tiled
  // kernel's
  tile_of_block<KS ? 8 : 4>(bx, by, bz);
  // K split (KS): both groups take the same rows and alternate K steps
  const int64_t m_base = KS ? (int64_t)bx * GM : (int64_t)bx * (2 * GM) + grp * GM;
  const int64_t NB = p.N >> 4;
  const int64_t nb_base = (int64_t)by * 16 + gw * NT;
  const int KB = (int)(p.K >> 7);
  const int kb0 = (int)((int64_t)KB * bz / splitk);
  const int kb1 = (int)((int64_t)KB * (bz + 1) / splitk);
  const int kb_first = KS ? kb0 + grp : kb0;   // this group's first K step

  const int64_t rows_valid = p.M - m_base < GM ? p.M - m_base : GM;
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(static_cast<const uint8_t*>(p.a) + (rows_valid > 0 ? m_base * p.K : 0), rows_valid * p.K);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(reinterpret_cast<const uint8_t*>(p.b) + (nb_base < NB ? nb_base * KB * 1024 : 0),
                (NB - nb_base) * KB * 1024);

  uint32_t a_off[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int row = (4 * j + gw) * RPL + lane / CPR;
    const int chunk = (lane % CPR) ^ lds_swizzle<1>(row);
    a_off[j] = (uint32_t)(row * p.K + chunk * 16);
  }
  uint8_t* const my_lds = lds + grp * HALF;
  auto load_a = [&](int kb, int st) {
    const uint32_t base = kb < kb1 ? (uint32_t)(kb * ROWB) : kOutOfRange;
#pragma unroll
    for (int j = 0; j < LPT; ++j)
      buffer_load_lds16(ra, my_lds + st * STAGE + (4 * j + gw) * RPL * ROWB, base + a_off[j]);
  };
  auto load_w = [&](int kb, u32x4* w) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      w[nt] = buffer_load16(rw, kb < kb1 ? (uint32_t)(((nt * KB) + kb) * 1024 + lane * 16) : kOutOfRange);
  };
  int frag_off[AV];
#pragma unroll
  for (int j = 0; j < AV; ++j) frag_off[j] = r * ROWB + (((kq * AV + j) ^ lds_swizzle<1>(r)) * 16);

  Acc acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = Acc{};
  uint32_t e[NT][16];

  // V: wait for the step's own loads, expand its weights, issue the loads of
  // step kb + 2 (weights into the registers just expanded, tile into the
  // stage step kb - 1 used).
  auto phase_v = [&](int kb, u32x4* w) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kAfter));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(w[nt]));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) expand_weights<OP, FLIP>(w[nt], f16x2{}, e[nt]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pin_words<kExpandedWords<OP>>(e[nt]);
    load_w(kb + 2 * STRIDE, w);
    load_a(kb + 2 * STRIDE, ((kb - kb_first) / STRIDE + 2) % 3);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // M: the step's MFMAs on its stage.
  auto phase_m = [&](int kb) {
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* src = my_lds + (((kb - kb_first) / STRIDE) % 3) * STAGE;
    u32x4 af[MT][AV];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < AV; ++j) af[mt][j] = *reinterpret_cast<const u32x4*>(src + mt * 16 * ROWB + frag_off[j]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) block_mma<OP>(e[nt], af[mt], acc[nt][mt]);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * AV, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      __builtin_amdgcn_sched_group_barrier(0x008, NT * kMfmaPerBlock<OP>, 0);
      if (mt + 2 < MT) __builtin_amdgcn_sched_group_barrier(0x100, AV, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto bar = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  u32x4 w0[NT], w1[NT];
  load_a(kb_first, 0);
  load_w(kb_first, w0);
  asm volatile("" ::: "memory");
  load_a(kb_first + STRIDE, 1);
  load_w(kb_first + STRIDE, w1);
  asm volatile("" ::: "memory");

  // Slots separated by workgroup barriers.  Every wave runs V(kb) M(kb)
  // V(kb+1) M(kb+1) ..., one slot per barrier; group 1 starts one barrier
  // later (and group 0 ends with one more), so in every slot one group issues
  // its MFMAs while the other expands and loads.  Both groups pass the same
  // number of barriers.
  // steps per group: with the K split both groups take the same count (group
  // 1's last step may lie past the range: its loads read zeros)
  const int n = KS ? (kb1 - kb0 + 1) / 2 : kb1 - kb0;
  if (grp == 1) bar();
  int kb = kb_first;
  for (int pairs = n >> 1; pairs > 0; --pairs, kb += 2 * STRIDE) {
    bar();
    phase_v(kb, w0);
    bar();
    phase_m(kb);
    bar();
    phase_v(kb + STRIDE, w1);
    bar();
    phase_m(kb + STRIDE);
  }
  if (n & 1) {
    bar();
    phase_v(kb, w0);
    bar();
    phase_m(kb);
  }
  if (grp == 0) bar();
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  if constexpr (KS) {
    // the halves' sum (exact int32) through LDS: group 1 stores its
    // accumulators, group 0 adds them and runs the epilogue.  Wave gw of
    // either group owns the same columns; quad q of lane l is at
    // ((gw * 32 + q) * 64 + l) * 16 (each store fills 1 KiB, conflict-free).
    __syncthreads();   // every wave is done with the ring
    i32x4* red = reinterpret_cast<i32x4*>(lds);
    if (grp == 1) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[(gw * NT * MT + nt * MT + mt) * 64 + lane] = acc[nt][mt];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] += red[(gw * NT * MT + nt * MT + mt) * 64 + lane];
  }

  // Epilogue (as the tiled kernel's, per channel).
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t n_d = (nb_base + nt) * 16 + 4 * kq;
    if (n_d >= p.N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = m_base + mt * 16 + r;
      if (m >= p.M) continue;
      uint32_t bits[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bits[i] = (uint32_t)acc[nt][mt][i];
      if constexpr (SPLIT) {
        uint32_t* slot = static_cast<uint32_t*>(p.ws) + ((int64_t)bz * p.M + m) * p.N + n_d;
        *reinterpret_cast<u32x4*>(slot) = u32x4{bits[0], bits[1], bits[2], bits[3]};
      } else if constexpr (PARTIALS) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (in_window(p, m, n_d + i))
            store_partial<OP>(p, 0, m, n_d + i, __uint_as_float(bits[i]), (int32_t)bits[i] >> 4);
      } else {
        uint16_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = finalize<OP, false>(p, m, n_d + i, __uint_as_float(bits[i]), (int32_t)bits[i]);
          o[i] = p.out_dtype == W4_F16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
        }
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + m * p.N + n_d) =
            make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
      }
    }
  }
}

template <bool KS>
static hipError_t launch_rows(const GemmArgs& args, bool flip, const GemmPlan& plan, hipStream_t stream) {
  const int64_t BM = KS ? 128 : 256;
  const dim3 grid((unsigned)((args.M + BM - 1) / BM), (unsigned)((args.N + 255) / 256), (unsigned)plan.splitk);
  const bool part = args.mode == MODE_PARTIALS;
  if (plan.splitk > 1) {
    if (flip) hipLaunchKernelGGL((w4_gemm_pingpong<KS, true, true, false>), grid, dim3(512), 0, stream, args, plan.splitk);
    else hipLaunchKernelGGL((w4_gemm_pingpong<KS, false, true, false>), grid, dim3(512), 0, stream, args, plan.splitk);
  } else if (part) {
    if (flip) hipLaunchKernelGGL((w4_gemm_pingpong<KS, true, false, true>), grid, dim3(512), 0, stream, args, 1);
    else hipLaunchKernelGGL((w4_gemm_pingpong<KS, false, false, true>), grid, dim3(512), 0, stream, args, 1);
  } else {
    if (flip) hipLaunchKernelGGL((w4_gemm_pingpong<KS, true, false, false>), grid, dim3(512), 0, stream, args, 1);
    else hipLaunchKernelGGL((w4_gemm_pingpong<KS, false, false, false>), grid, dim3(512), 0, stream, args, 1);
  }
  return hipGetLastError();
}

hipError_t launch_pingpong(const GemmArgs& args, bool flip, const GemmPlan& plan, hipStream_t stream) {
  if (plan.bn != 256) return hipErrorInvalidValue;
  hipError_t e = plan.bm == 256 ? launch_rows<false>(args, flip, plan, stream)
                 : plan.bm == 128 ? launch_rows<true>(args, flip, plan, stream)
                                  : hipErrorInvalidValue;
  if (e != hipSuccess || plan.splitk == 1) return e;
  return launch_splitk_reduce(args, OP_I8, false, plan.splitk, stream);
}

}  // namespace w4
