// Streaming GEMM kernel for gfx950: the band of M where the packed weight
// stream bounds the W4A8 GEMM but the activations have outgrown the small-M
// kernel (8-bit operands, 16 < M <= 128).
//
//   out[m,n] = RNE( s_a[m] * sum_g s[n,g] * sum_{k in g} a[m,k] * w[n,k] + bias[n] )
//
// ("support W4A8 Marlin kernel": per-channel and per-group W4A8, which that
// PR's review finds memory-bound below a few hundred tokens; Machete README,
// "Overview".)
#include "w4_gemm_common.h"

namespace w4 {

// ===========================================================================
// Streaming kernel: the band of M where the weight stream still bounds the
// GEMM but the activations no longer fit the small-M kernel's fragments
// (8-bit operands, 16 < M <= 128).
//
// Same tile shape as the tiled kernel (BM = 16 MT rows, 4 waves, wave w owns
// NT 16-column n-blocks), but the weight blocks of each 128-deep K step go
// straight from memory into LDS next to the activation tile, and the ring
// holds STAGES steps: STAGES - 1 steps of weights are in flight per wave,
// where the tiled kernel keeps its weights in registers and has at most two
// steps in flight.  Bytes in flight, not arithmetic, bound this band: one
// 128-deep step of a 64 x 256 tile is 32 MFMAs per wave, far shorter than a
// memory round trip.  Each wave reads back only its own weight blocks; the
// block lands in LDS in lane order, so the read is conflict-free.  A grouped
// problem's scales for the workgroup's K range and columns are staged once
// into an LDS table at the start ([group][column], fp32, int8 scales times
// 1/16).
//
// Per step: one barrier (every wave's loads of this step have landed and
// every wave has finished reading the stage the next loads overwrite), then
// the loads of step kb + STAGES - 1 into the stage step kb - 1 used, then
// this step's MFMAs.  Loads past the K range read zeros and move no data, so
// every step issues the same number of loads and the wait count is exact.
// ===========================================================================
template <int MT, int NT, int STAGES>
struct StreamShape {
  static constexpr int BM = MT * 16;
  static constexpr int ASTAGE = BM * 128;            // activation tile bytes (8-bit rows of 128 k)
  static constexpr int WSTAGE = 4 * NT * 1024;       // the four waves' weight blocks
  static constexpr int STAGE = ASTAGE + WSTAGE;
  static constexpr int BNW = 4 * NT * 16;            // columns of the workgroup
  static constexpr int TABG = stream_table_groups(BNW);   // groups the 32 KiB scale table holds
  static constexpr int TAB = TABG * BNW * 4;
  static constexpr int LDS = STAGES * STAGE;         // plus TAB when grouped
};

template <int OP, bool GROUPED, bool FLIP, int NT, int MT, int STAGES, bool SPLIT, bool PARTIALS>
__global__ __launch_bounds__(256, 1) void w4_gemm_stream(GemmArgs p, int splitk) {
  static_assert(OP == OP_I8 || OP == OP_FP8, "8-bit operands");
  static_assert(MT >= 2 && MT % 2 == 0, "tile rows: a multiple of 32");
  using Acc = typename OpTraits<OP>::Acc;
  using Shape = StreamShape<MT, NT, STAGES>;
  constexpr int EB = 1;
  constexpr int AV = act_vecs<OP>();          // 2 16-byte words per lane per fragment
  constexpr int ROWB = 128;
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  constexpr int RPL = 1024 / ROWB;            // rows one wave-wide 16-byte load fills
  constexpr int LPT = Shape::BM / (4 * RPL);  // activation loads per wave per step
  constexpr int LPS = LPT + NT;               // loads per wave per step
  constexpr bool kFold = GROUPED && !PARTIALS;
  constexpr int BNW = Shape::BNW;
  static_assert((STAGES - 2) * LPS <= 63, "the wait count must fit vmcnt");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Shape::LDS + (kFold ? Shape::TAB : 0)];
  float* const tab = reinterpret_cast<float*>(lds + Shape::LDS);   // [group - kb0][column]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int kq = lane >> 4;
  int bx, by, bz;
  tile_of_block(bx, by, bz);
  const int64_t m_base = (int64_t)bx * Shape::BM;
  const int64_t NB = p.N >> 4;
  const int64_t nb_base = (int64_t)by * (4 * NT) + wave * NT;
  const int KB = (int)(p.K >> 7);
  const int kb0 = (int)((int64_t)KB * bz / splitk);
  const int kb1 = (int)((int64_t)KB * (bz + 1) / splitk);
  constexpr bool partials = PARTIALS;

  const int64_t rows_valid = p.M - m_base < Shape::BM ? p.M - m_base : Shape::BM;
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(static_cast<const uint8_t*>(p.a) + m_base * p.K, rows_valid * p.K);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(reinterpret_cast<const uint8_t*>(p.b) + nb_base * KB * 1024, (NB - nb_base) * KB * 1024);
  const int sbytes = p.s_dtype == W4_F32 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.s, (int64_t)(p.s != nullptr) * p.N * p.G * sbytes);

  // Load j of this wave fills tile rows [(4 j + wave) RPL, +RPL) (swizzled
  // chunks, as in the tiled kernel).
  uint32_t a_off[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int row = (4 * j + wave) * RPL + lane / CPR;
    const int chunk = (lane % CPR) ^ lds_swizzle<EB>(row);
    a_off[j] = (uint32_t)(row * p.K + chunk * 16);
  }
  auto issue = [&](int kb, int st) {
    uint8_t* const base = lds + st * Shape::STAGE;
    const uint32_t abase = kb < kb1 ? (uint32_t)(kb * ROWB) : kOutOfRange;
#pragma unroll
    for (int j = 0; j < LPT; ++j) buffer_load_lds16(ra, base + (4 * j + wave) * RPL * ROWB, abase + a_off[j]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      buffer_load_lds16(rw, base + Shape::ASTAGE + (wave * NT + nt) * 1024,
                        kb < kb1 ? (uint32_t)((nt * KB + kb) * 1024 + lane * 16) : kOutOfRange);
  };

  Acc acc[NT][MT];
  f32x4 tot[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[nt][mt] = Acc{};
      tot[nt][mt] = f32x4{};
    }
  int frag_off[AV];
#pragma unroll
  for (int j = 0; j < AV; ++j) frag_off[j] = r * ROWB + (((kq * AV + j) ^ lds_swizzle<EB>(r)) * 16);

  // Grouped: the scale table of the K range, staged while the ring's first
  // steps are in flight.  Thread t takes column t % BNW and groups
  // kb0 + t / BNW + i (256 / BNW), in rounds of 8.
  const int col = tid % BNW;
  const uint32_t col_n = (uint32_t)((int64_t)by * BNW + col);
  const int gfirst = tid / BNW;
  constexpr int GSTEP = 256 / BNW;
  uint32_t tw[8];
  auto tab_load = [&](int g0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = kb0 + g0 + gfirst + i * GSTEP;
      tw[i] = load_word(rs, p.s_dtype, col_n * (uint32_t)p.G + (uint32_t)g, g < kb1 && col_n < (uint32_t)p.N);
    }
  };
  auto tab_store = [&](int g0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int gl = g0 + gfirst + i * GSTEP;   // group relative to kb0
      if (gl < Shape::TABG) {
        float sv = word_to_f32(tw[i], p.s_dtype, col_n * (uint32_t)p.G + (uint32_t)(kb0 + gl));
        if constexpr (OP == OP_I8) sv *= 0.0625f;   // the operand holds 16 w
        tab[gl * BNW + col] = sv;
      }
    }
  };

  // One K step from stage st.
  auto step = [&](int kb, int st) {
    const uint8_t* const base = lds + st * Shape::STAGE;
    uint32_t e[NT][16];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(base + Shape::ASTAGE + (wave * NT + nt) * 1024 + lane * 16);
      expand_weights<OP, FLIP>(w, f16x2{}, e[nt]);
    }
    u32x4 af[MT][AV];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < AV; ++j)
        af[mt][j] = *reinterpret_cast<const u32x4*>(base + mt * 16 * ROWB + frag_off[j]);
    if constexpr (kFold) {
      const int gl = kb - kb0;
      f32x4 scv[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        scv[nt] = *reinterpret_cast<const f32x4*>(&tab[gl * BNW + (wave * NT + nt) * 16 + 4 * kq]);
      auto fold_block = [&](int nt, int mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = (OP == OP_I8) ? (float)acc[nt][mt][i] : (float)acc[nt][mt][i];
          tot[nt][mt][i] = fmaf(pv, scv[nt][i], tot[nt][mt][i]);
        }
      };
      // row mt's MFMAs start from zero; row mt - 1 is folded while they run
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          Acc t = Acc{};
          block_mma<OP>(e[nt], af[mt], t);
          acc[nt][mt] = t;
          if (mt > 0) fold_block(nt, mt - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) fold_block(nt, MT - 1);
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) block_mma<OP>(e[nt], af[mt], acc[nt][mt]);
    }
    if constexpr (GROUPED && PARTIALS) {
      // verification mode: store each group's dot products
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int64_t n_d = (nb_base + nt) * 16 + 4 * kq;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int64_t m = m_base + mt * 16 + r;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (m < p.M && n_d < p.N && in_window(p, m, n_d + i))
              store_partial<OP>(p, kb, m, n_d + i, partial_value<OP>(acc[nt][mt], f32x4{}, 0.0f, i),
                                int_partial<OP>(acc[nt][mt], i));
          acc[nt][mt] = Acc{};
        }
      }
    }
  };

  // Prologue: the table's first round, then the first STAGES - 1 steps.
  const int nsteps = kb1 - kb0;
  if constexpr (kFold) tab_load(0);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int s0 = 0; s0 < STAGES - 1; ++s0) issue(kb0 + s0, s0);
  asm volatile("" ::: "memory");
  if constexpr (kFold) {
    tab_store(0);
    for (int g0 = 8 * GSTEP; g0 < nsteps; g0 += 8 * GSTEP) {
      tab_load(g0);
      tab_store(g0);
    }
  }
  int st = 0;
  for (int kb = kb0; kb < kb1; ++kb) {
    stage_barrier<(STAGES - 2) * LPS>();
    issue(kb + STAGES - 1, st == 0 ? STAGES - 1 : st - 1);
    asm volatile("" ::: "memory");
    step(kb, st);
    st = st == STAGES - 1 ? 0 : st + 1;
  }
  // drain the loads issued past the last step before the LDS is released
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

  if (GROUPED && partials) return;
  // Epilogue (as the tiled kernel's).
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
      for (int i = 0; i < 4; ++i) {
        if constexpr (GROUPED)
          bits[i] = __float_as_uint(tot[nt][mt][i]);
        else if constexpr (OP == OP_I8)
          bits[i] = (uint32_t)acc[nt][mt][i];
        else
          bits[i] = __float_as_uint(partial_value<OP>(acc[nt][mt], f32x4{}, 0.0f, i));
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


template <int OP, bool GROUPED, bool FLIP, int MT, int NT, int STAGES>
static hipError_t launch_shape(const GemmArgs& args, const GemmPlan& plan, hipStream_t stream) {
  const int64_t BM = MT * 16, BN = NT * 64;
  const dim3 grid((unsigned)((args.M + BM - 1) / BM), (unsigned)((args.N + BN - 1) / BN), (unsigned)plan.splitk);
  const bool part = args.mode == MODE_PARTIALS;
  if (plan.splitk > 1) {
    if (part)
      hipLaunchKernelGGL((w4_gemm_stream<OP, GROUPED, FLIP, NT, MT, STAGES, true, true>), grid, dim3(256), 0, stream,
                         args, plan.splitk);
    else
      hipLaunchKernelGGL((w4_gemm_stream<OP, GROUPED, FLIP, NT, MT, STAGES, true, false>), grid, dim3(256), 0, stream,
                         args, plan.splitk);
  } else {
    if (part)
      hipLaunchKernelGGL((w4_gemm_stream<OP, GROUPED, FLIP, NT, MT, STAGES, false, true>), grid, dim3(256), 0, stream,
                         args, 1);
    else
      hipLaunchKernelGGL((w4_gemm_stream<OP, GROUPED, FLIP, NT, MT, STAGES, false, false>), grid, dim3(256), 0, stream,
                         args, 1);
  }
  hipError_t e = hipGetLastError();
  // grouped partials are stored by the kernel itself
  if (e != hipSuccess || plan.splitk == 1 || (GROUPED && part)) return e;
  return launch_splitk_reduce(args, OP, GROUPED, plan.splitk, stream);
}

template <int OP, bool GROUPED, bool FLIP>
static hipError_t launch_typed(const GemmArgs& args, const GemmPlan& plan, hipStream_t stream) {
  // tile shapes and ring depths (stream_stages)
  if (plan.bm == 32 && plan.bn == 256) return launch_shape<OP, GROUPED, FLIP, 2, 4, stream_stages(2, 4)>(args, plan, stream);
  if (plan.bm == 64 && plan.bn == 256) return launch_shape<OP, GROUPED, FLIP, 4, 4, stream_stages(4, 4)>(args, plan, stream);
  if (plan.bm == 128 && plan.bn == 128) return launch_shape<OP, GROUPED, FLIP, 8, 2, stream_stages(8, 2)>(args, plan, stream);
  if (plan.bm == 32 && plan.bn == 128) return launch_shape<OP, GROUPED, FLIP, 2, 2, stream_stages(2, 2)>(args, plan, stream);
  if (plan.bm == 64 && plan.bn == 128) return launch_shape<OP, GROUPED, FLIP, 4, 2, stream_stages(4, 2)>(args, plan, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_stream(const GemmArgs& args, int op, bool grouped, bool flip, const GemmPlan& plan,
                         hipStream_t stream) {
  if (args.x || args.z || args.prescaled_zeros) return hipErrorInvalidValue;
  if (op == OP_I8) {
    if (grouped) return flip ? launch_typed<OP_I8, true, true>(args, plan, stream) : launch_typed<OP_I8, true, false>(args, plan, stream);
    return flip ? launch_typed<OP_I8, false, true>(args, plan, stream) : launch_typed<OP_I8, false, false>(args, plan, stream);
  }
  if (op == OP_FP8) {
    if (grouped) return flip ? launch_typed<OP_FP8, true, true>(args, plan, stream) : launch_typed<OP_FP8, true, false>(args, plan, stream);
    return flip ? launch_typed<OP_FP8, false, true>(args, plan, stream) : launch_typed<OP_FP8, false, false>(args, plan, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace w4
