// C ABI of the 4-bit-weight GEMM library: argument validation, kernel
// selection and launch.  Validation runs entirely on the host and returns
// before any HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "w4.h"
#include "w4_internal.h"

namespace {

using namespace w4;

thread_local std::string g_last_error;

std::atomic<int64_t> g_force_path{0};
std::atomic<int64_t> g_splitk{0};
std::atomic<int64_t> g_norm_exact_sum{0};
std::atomic<int64_t> g_skinny_strips{0};
std::atomic<int64_t> g_tiled_bm{0};
std::atomic<int64_t> g_schedule_table{1};

// A kernel schedule: path, K split, tile rows (tiled kernel) and 16-column
// strips per wave (small-M kernel); 0 leaves a field to the heuristic.
struct Sched {
  int64_t path = 0, splitk = 0, tile_m = 0, strips = 0;
  bool any() const { return path || splitk || tile_m || strips; }
};

// Schedule table entry: problems of this activation type, grouping, N and K
// with m_lo <= M <= m_hi take this schedule.
struct SchedEntry {
  int a_dtype, grouped;
  int64_t N, K, m_lo, m_hi;
  int path, splitk, tile_m, strips;
};

// Built-in entries, measured on MI355X by the package's autotune module for
// the shapes of its benchmarks (only where they beat the heuristic); the last
// entry is a sentinel.
const SchedEntry kBuiltinSchedules[] = {
#include "w4_schedule_table.inc"
    {-1, 0, 0, 0, 0, 0, 0, 0, 0, 0},
};

std::mutex g_sched_mutex;
std::vector<SchedEntry> g_sched_user;   // entries added at run time, searched first

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return W4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_fail(hipError_t e, const char* what) {
  return fail(W4_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device, cached per device.  Falls back to the
// MI355X count when no device can be queried (planning-only calls on a host
// without a GPU).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
    (void)hipGetLastError();
    v = 256;
  }
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

int64_t resolve_group(int64_t group_size, int64_t K) { return group_size == -1 ? K : group_size; }

// Tile rows of the streaming kernel for 16 < M <= 64 (128-column tiles, one
// workgroup per CU): 32 up to M = 32, 64 above, or 64 when 32-row tiles would
// need more than one round of workgroups; 0 when even 64-row tiles would, and
// for grouped problems above M = 32 (the tiled kernel then: its 64 x 128
// tiles measured faster there on the grouped benchmark shapes).
int64_t stream_tile_m(int64_t M, int64_t N, bool grouped, int cu) {
  const int64_t cols = (N + 127) / 128;
  if (grouped && M > 32) return 0;   // the tiled kernel's 64 x 128 tiles
  int64_t bm = M <= 32 ? 32 : 64;
  if (bm == 32 && M > 32 && ((M + 31) / 32) * cols > cu) bm = 64;
  return ((M + bm - 1) / bm) * cols > cu ? 0 : bm;
}

int op_of(int a_dtype) {
  switch (a_dtype) {
    case W4_I8: return OP_I8;
    case W4_FP8_E4M3: return OP_FP8;
    case W4_F16: return OP_F16;
    case W4_BF16: return OP_BF16;
    default: return -1;
  }
}

int check_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0)
    return fail(W4_E_SHAPE, "need M >= 0, N > 0, K > 0 (got M=%lld N=%lld K=%lld)", (long long)M,
                (long long)N, (long long)K);
  if (N % 16) return fail(W4_E_SHAPE, "N=%lld must be a multiple of 16", (long long)N);
  if (K % 128) return fail(W4_E_SHAPE, "K=%lld must be a multiple of 128", (long long)K);
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30)
    return fail(W4_E_SHAPE, "sizes above 2^30 are not supported");
  return W4_OK;
}

// W4A16 (small_ok) also takes groups of 64 and 32.
int check_group(int64_t group_size, int64_t K, bool small_ok = false) {
  const int64_t g = resolve_group(group_size, K);
  if (g != K && g != 128 && !(small_ok && (g == 64 || g == 32)))
    return fail(W4_E_GROUP, "group_size=%lld: supported values are K, -1 and 128%s", (long long)group_size,
                small_ok ? ", 64, 32" : "");
  if (K % g) return fail(W4_E_GROUP, "group_size=%lld does not divide K=%lld", (long long)g, (long long)K);
  return W4_OK;
}

// Kernel choice.  Small M is bound by the weight stream and uses the skinny
// kernel with enough K-splitting waves to keep ~16 waves per CU in flight;
// larger M uses the tiled kernel, split along K while there are fewer tiles
// than CUs.  Fields of `forced` that are nonzero replace the heuristic's
// choice (and must fit the problem).  zp: asymmetric int8, whose small-M
// kernel keeps a second (zero-point) table.
int plan_with(int64_t M, int64_t N, int64_t K, bool grouped, int op, const Sched& forced, GemmPlan* plan,
              bool zp = false, int sg = 1) {
  // The kernels address a tile's activation rows (up to 256 of them), a
  // wave's weight blocks and the scale / zero-point tables with 32-bit buffer
  // offsets into ranges of at most 2 GiB.
  if (K > ((int64_t)1 << 22)) return fail(W4_E_SHAPE, "GEMMs with K=%lld above 2^22 are not supported", (long long)K);
  if (N * (grouped ? (K / 128) * sg : 1) > ((int64_t)1 << 29) - 4)
    return fail(W4_E_SHAPE, "GEMMs with more than 2^29 - 4 scales (N x groups) are not supported");
  const int64_t fp = forced.path, fs = forced.splitk;
  const int64_t KB = K / 128;
  const int cu = cu_count();
  // small M: the small-M kernel; 16 < M <= 64 with symmetric int8 (grouped:
  // M <= 32): the streaming kernel (measured faster on every int8 benchmark
  // shape at M = 32 and per channel at M = 64; fp8, whose lookup expansion
  // keeps one wave per SIMD busy, is faster tiled); larger M: the tiled kernel
  const bool stream_ok = op == OP_I8 && !zp && sg == 1 && M > 16 && M <= 64 && stream_tile_m(M, N, grouped, cu);
  // symmetric int8 per channel: the ping-pong kernel (one eight-wave
  // workgroup per CU whose two halves take turns on the MFMAs), K split by
  // the largest power of two that keeps the workgroups within one per CU,
  // once its workgroups occupy 3/4 of the CUs or more and come in whole
  // rounds of one per CU (a partial last round leaves CUs idle for a whole
  // tile's time; the tiled kernel, two smaller workgroups per CU, loses less
  // there).  256 x 256 tiles when they need at most two K splits for that
  // (8192 x 21760: 4-5% faster than two tiled workgroups per CU at M =
  // 2048-8192; M = 576-768 with two splits 114-118 against 128-130 us; at
  // M = 3072, 1.5 rounds, 488 against 431 us tiled); else 128 x 256 tiles
  // whose halves split K between them, within one round, with at most 4 K
  // splits (M = 384 and 512 with two splits: 70 and 79 against 80 and 85 us
  // tiled; 256 x 256 tiles with four splits took 113 us at M = 512; at M =
  // 1280, 1.25 rounds, 273 against 219 us tiled); a forced 256-row tile
  // selects it too
  const bool pc8 = op == OP_I8 && !grouped && !zp && sg == 1;
  auto pp_split = [&](int64_t tiles, int64_t smax) {
    int64_t s = 1;
    while (s * 2 <= smax && tiles * s * 2 <= cu) s *= 2;
    return s;
  };
  const int64_t pp_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t pp_ks_tiles = ((M + 127) / 128) * ((N + 255) / 256);
  const int64_t pp_w256 = pp_tiles * pp_split(pp_tiles, 8);       // workgroups
  const int64_t pp_w128 = pp_ks_tiles * pp_split(pp_ks_tiles, 4);
  const bool pp_256 = pp_w256 <= 2 * pp_tiles && 4 * pp_w256 >= 3LL * cu && (pp_w256 <= cu || pp_w256 % cu == 0);
  const bool pp_auto = pp_256 || (4 * pp_w128 >= 3LL * cu && pp_w128 <= cu);
  const bool pp_ok = pc8 && M > 64 && (forced.tile_m == 256 || (!forced.tile_m && !forced.strips && pp_auto));
  plan->path = fp ? (int)fp
                  : (M <= 16 ? PATH_SKINNY : stream_ok ? PATH_STREAM : pp_ok ? PATH_PINGPONG : PATH_TILED);
  tiled_tile(op, grouped, 0, &plan->bm, &plan->bn, zp);
  // strips of 16 columns per wave of the small-M kernel: two strips share
  // one activation fragment.  Grouped problems take two when N leaves enough
  // workgroups and either the fragment is worth sharing (M >= 8) or the
  // strips are long (K >= 8192) or many (N >= 16384): a wave then keeps
  // twice the weight bytes in flight.
  const int64_t fns = plan->path == PATH_SKINNY ? forced.strips : 0;
  if (plan->path == PATH_SKINNY && fns > 2) return fail(W4_E_SHAPE, "small-M kernel: 1 or 2 strips per wave");
  const bool two = N % 32 == 0 && (!grouped || N >= 16384 || (N >= 8192 && (M >= 8 || KB >= 64)));
  int64_t ns = fns ? fns : (two ? 2 : 1);
  const int64_t groups = grouped ? KB * sg : 1;   // sg groups per 128-deep block
  bool one_split = false;
  if (plan->path == PATH_SKINNY && skinny_table_bytes(op, grouped, groups, (int)ns, zp) > kSkinnyTableMax) {
    // the scale / zero-point tables would not fit the small-M kernel's LDS
    if (!fns && ns == 2 && skinny_table_bytes(op, grouped, groups, 1, zp) <= kSkinnyTableMax) {
      ns = 1;
    } else if (fp || fns) {
      return fail(W4_E_UNSUPPORTED, "the small-M kernel's LDS tables do not fit K=%lld", (long long)K);
    } else {
      plan->path = PATH_TILED;
      // where only the zero-point table tips the balance, the symmetric plan
      // (whose workspace size callers query) has none: no K split either
      one_split = zp && skinny_table_bytes(op, grouped, groups, 1) <= kSkinnyTableMax;
    }
  }
  if (plan->path == PATH_PINGPONG) {
    // ping-pong kernel: symmetric int8 per channel, 256 rows (two 128-row
    // halves) or 128 rows (two halves splitting K) x 256 columns, one
    // workgroup per CU
    if (!pc8) return fail(W4_E_UNSUPPORTED, "the ping-pong kernel takes symmetric int8 per channel");
    const int64_t fbm = forced.tile_m;
    if (fbm && fbm != 128 && fbm != 256)
      return fail(W4_E_SHAPE, "ping-pong kernel: tile rows 128 or 256 (got %lld)", (long long)fbm);
    if (forced.strips && forced.strips != 4)
      return fail(W4_E_SHAPE, "ping-pong kernel: tiles are 256 columns wide (4 column blocks per wave)");
    plan->bm = (int)(fbm ? fbm : (pp_256 ? 256 : 128));
    plan->bn = 256;
    const int64_t tiles = ((M + plan->bm - 1) / plan->bm) * ((N + 255) / 256);
    int64_t s = fs;
    if (!s) {
      s = pp_split(tiles, plan->bm == 128 ? 4 : 8);
      while (s > 1 && KB / s < 4) s /= 2;
    }
    if (s < 1 || s > 64 || s > KB)
      return fail(W4_E_SHAPE, "ping-pong kernel: K split %lld not in [1, min(64, K/128)]", (long long)s);
    plan->splitk = (int)s;
    return W4_OK;
  }
  if (plan->path == PATH_STREAM) {
    // streaming kernel: 8-bit symmetric operands, one workgroup per CU
    if ((op != OP_I8 && op != OP_FP8) || zp || sg != 1)
      return fail(W4_E_UNSUPPORTED, "the streaming kernel takes int8 / fp8 activations and symmetric weights");
    const int64_t fbm = forced.tile_m;
    if (fbm && fbm != 32 && fbm != 64 && fbm != 128)
      return fail(W4_E_SHAPE, "streaming kernel: tile rows 32, 64 or 128 (got %lld)", (long long)fbm);
    int64_t bm = fbm;
    if (!bm) {
      bm = M <= 64 ? stream_tile_m(M, N, grouped, cu) : 128;
      if (!bm) bm = M <= 32 ? 32 : 64;   // forced onto a problem with more tiles than CUs
    }
    // 16-column blocks per wave (the strips field): 2 (the default: more
    // column tiles, fewer K splits) or 4; 128-row tiles take 2
    const int64_t fnt = forced.strips;
    if (fnt && fnt != 2 && fnt != 4) return fail(W4_E_SHAPE, "streaming kernel: 2 or 4 column blocks per wave");
    if (bm == 128 && fnt == 4) return fail(W4_E_SHAPE, "streaming kernel: 128-row tiles take 2 column blocks per wave");
    plan->bm = (int)bm;
    plan->bn = (int)(64 * (fnt ? fnt : 2));
    const int64_t tiles = ((M + plan->bm - 1) / plan->bm) * ((N + plan->bn - 1) / plan->bn);
    int64_t s = fs;
    if (!s) {
      s = tiles >= cu ? 1 : cu / tiles;
      if (s > 64) s = 64;
      while (s > 1 && KB / s < 2) --s;
    }
    // a grouped split's scales must fit the kernel's table
    const int tg = stream_table_groups(plan->bn);
    if (grouped && (KB + s - 1) / s > tg) {
      if (fs) return fail(W4_E_SHAPE, "streaming kernel: %lld K splits leave more than %d groups per split",
                          (long long)s, tg);
      s = (KB + tg - 1) / tg;
    }
    if (s < 1 || s > 64 || s > KB)
      return fail(W4_E_SHAPE, "streaming kernel: K split %lld not in [1, min(64, K/128)]", (long long)s);
    plan->splitk = (int)s;
    return W4_OK;
  }
  if (plan->path == PATH_SKINNY) {
    if (M > 16) return fail(W4_E_UNSUPPORTED, "the small-M kernel handles M <= 16 (M=%lld)", (long long)M);
    if (N % (16 * ns))
      return fail(W4_E_SHAPE, "small-M kernel with %lld strips per wave needs N %% %lld == 0", (long long)ns,
                  (long long)(16 * ns));
    plan->bn = (int)(16 * ns);
    int64_t s;
    if (fs) {
      s = fs;
    } else {
      // ~16 resident waves per CU, each with at least 8 weight blocks (K
      // blocks times strips; shorter waves spend most of their time waiting
      // for their first loads)
      const int64_t groups = N / (16 * ns);
      const int64_t want = (16 * cu + groups - 1) / groups;
      s = 1;
      while (s < want && s < 8) s *= 2;
      while (s > 1 && KB * ns / s < 8) s /= 2;
    }
    const int smax = skinny_max_waves(op, grouped);
    if (s < 1 || s > smax || s > KB)
      return fail(W4_E_SHAPE, "small-M kernel: %lld K-splitting waves not in [1, min(%d, K/128)]", (long long)s,
                  smax);
    plan->splitk = (int)s;
  } else {
    // 8-bit operands: 128-row tiles when there are enough of them (int8
    // per channel: one workgroup per CU, with K splits up to two per CU
    // (8192 x 21760 M = 1280: 219 us, against 253 with 64 x 256 tiles);
    // its zero-point form: two; grouped int8, whose tall tile is 128 x 128:
    // one; grouped fp8: half a workgroup per CU once M fills the 128 rows),
    // 64 x 256 tiles otherwise
    const bool byte = op == OP_I8 || op == OP_FP8;
    const bool fp8g = op == OP_FP8 && grouped;
    const int64_t fbm = forced.tile_m;
    if (fbm == 32 || fbm == 256)
      return fail(W4_E_SHAPE, "tiled_bm=%lld is for the %s kernel", (long long)fbm, fbm == 32 ? "streaming" : "ping-pong");
    if (byte) {
      int tall_bm, tall_bn;
      tiled_tile(op, grouped, 1, &tall_bm, &tall_bn, zp);
      const int64_t tall_tiles = ((M + tall_bm - 1) / tall_bm) * ((N + tall_bn - 1) / tall_bn);
      const int64_t need = (op == OP_I8 && !grouped && zp) ? 2LL * cu : (int64_t)cu;
      const bool tall = fbm ? fbm == 128 : (fp8g ? M >= 128 && 2 * tall_tiles >= cu : tall_tiles >= need);
      tiled_tile(op, grouped, tall ? 1 : 0, &plan->bm, &plan->bn, zp);
      // grouped int8: 64 x 128 tiles while there are at most three per CU
      // (two workgroups per CU, half the per-group fold work per wave and
      // step of a 64 x 256 tile; measured faster than both other tiles on the
      // 7B-layer shapes from M = 33 to 512-1024), for long K (> 8192, where
      // 128 x 128 tiles with K splits win from M = 256) up to M = 128
      const int64_t narrow_tiles = ((M + 63) / 64) * ((N + 127) / 128);
      if (!fbm && op == OP_I8 && grouped && !zp && (K <= 8192 || M <= 128) && narrow_tiles <= 3LL * cu) {
        plan->bm = 64;
        plan->bn = 128;
      }
      // 16-column blocks per wave (the strips field): 2 (tiles of 128
      // columns) or 4 (256 columns: 64-row tiles, and 128-row tiles of
      // symmetric int8 per channel)
      const int64_t fnt = forced.strips;
      if (fnt) {
        if (fnt != 2 && fnt != 4) return fail(W4_E_SHAPE, "tiled kernel: 2 or 4 column blocks per wave");
        if (fnt == 4 && plan->bm == 128 && !(op == OP_I8 && !grouped && !zp))
          return fail(W4_E_SHAPE, "tiled kernel: 128 x 256 tiles are for symmetric int8 per channel");
        plan->bn = (int)(64 * fnt);
      }
    } else if (forced.strips && forced.strips != 2) {
      return fail(W4_E_SHAPE, "tiled kernel: 16-bit activations take 128-column tiles (2 blocks per wave)");
    } else if (fbm && fbm != plan->bm) {
      return fail(W4_E_SHAPE, "tiled_bm=%lld is not available for this problem", (long long)fbm);
    }
    int64_t s;
    if (fs) {
      s = fs;
    } else if (one_split) {
      s = 1;
    } else {
      // K splits: the fewest that give two workgroups per CU, or one per CU
      // when there are very few tiles (each split adds an M x N fp32 slot
      // that the reduce reads back, which outweighs the second workgroup
      // there).  Grouped int8 keeps the VALU busy with its per-group fold,
      // so a second workgroup per CU gains nothing: the most splits that
      // still fit one workgroup per CU.  Grouped fp8 (lookup expansion and
      // fold): the most that fit two.
      const int64_t tiles = ((M + plan->bm - 1) / plan->bm) * ((N + plan->bn - 1) / plan->bn);
      s = 1;
      if (op == OP_I8 && grouped) {
        while (tiles * s * 2 <= cu && s * 2 <= 16) s *= 2;
      } else if (fp8g) {
        while (tiles * s * 2 <= 2LL * cu && s * 2 <= 16) s *= 2;
      } else {
        const int64_t target = tiles < cu / 2 ? cu : 2LL * cu;
        while (tiles * s < target && s * 2 <= 8) s *= 2;
      }
      while (s > 1 && KB / s < 4) s /= 2;
    }
    if (s < 1 || s > 64 || s > KB)
      return fail(W4_E_SHAPE, "tiled kernel: K split %lld not in [1, min(64, K/128)]", (long long)s);
    plan->splitk = (int)s;
  }
  return W4_OK;
}

bool schedule_matches(const SchedEntry& e, int op, bool grouped, int64_t M, int64_t N, int64_t K) {
  return op_of(e.a_dtype) == op && (e.grouped != 0) == grouped && e.N == N && e.K == K && e.m_lo <= M &&
         M <= e.m_hi;
}

// Run-time entries first, then the built-in ones.
bool lookup_schedule(int op, bool grouped, int64_t M, int64_t N, int64_t K, Sched* out) {
  {
    std::lock_guard<std::mutex> lock(g_sched_mutex);
    for (const SchedEntry& e : g_sched_user)
      if (schedule_matches(e, op, grouped, M, N, K)) {
        *out = Sched{e.path, e.splitk, e.tile_m, e.strips};
        return true;
      }
  }
  for (const SchedEntry& e : kBuiltinSchedules) {
    if (e.a_dtype < 0) break;
    if (schedule_matches(e, op, grouped, M, N, K)) {
      *out = Sched{e.path, e.splitk, e.tile_m, e.strips};
      return true;
    }
  }
  return false;
}

// The options, when any is set, force their fields.  Otherwise a matching
// schedule-table entry (run-time entries first, then the built-in ones) is
// taken if it fits the problem, and the heuristic decides the rest.
int make_plan(int64_t M, int64_t N, int64_t K, bool grouped, int op, GemmPlan* plan, bool zp = false,
              int sg = 1) {
  const Sched opts{g_force_path.load(), g_splitk.load(), g_tiled_bm.load(), g_skinny_strips.load()};
  if (opts.any()) return plan_with(M, N, K, grouped, op, opts, plan, zp, sg);
  // the table's entries were measured with groups of 128
  if (g_schedule_table.load() && sg == 1) {
    Sched t;
    if (lookup_schedule(op, grouped, M, N, K, &t) && plan_with(M, N, K, grouped, op, t, plan, zp) == W4_OK)
      return W4_OK;
  }
  return plan_with(M, N, K, grouped, op, Sched{}, plan, zp, sg);
}

// Groups per 128-deep block (1 for 128 and per channel, 2 or 4 for 64 or 32).
int subgroups(int64_t group_size, int64_t K) {
  const int64_t g = resolve_group(group_size, K);
  return (g == 64 || g == 32) && g != K ? (int)(128 / g) : 1;
}

size_t workspace_for(const GemmPlan& plan, int64_t M, int64_t N) {
  if (plan.path == PATH_SKINNY || plan.splitk <= 1) return 0;
  return (size_t)plan.splitk * (size_t)M * (size_t)N * 4u;
}

// Shared front end of the GEMM entry points.
int run_gemm(GemmArgs& args, int op, bool grouped, bool flip, void* workspace, size_t workspace_bytes,
             void* stream, bool zp = false) {
  GemmPlan plan;
  const int sg = grouped ? (int)(128 * (int64_t)args.G / args.K) : 1;
  if (int st = make_plan(args.M, args.N, args.K, grouped, op, &plan, zp, sg)) return st;
  const size_t need = workspace_for(plan, args.M, args.N);
  if (need) {
    if (!workspace || workspace_bytes < need)
      return fail(W4_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(W4_E_ALIGN, "workspace must be 16-byte aligned");
  }
  args.ws = workspace;
  if (args.M == 0) return ok();
  hipError_t e = launch_gemm(args, op, grouped, flip, zp, plan, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "GEMM launch");
  return ok();
}

// Split-K workspace of w4a8_gemm_no_alloc, for callers that cannot allocate.
// One copy per GPU, held until the process ends; every call on a GPU shares
// it (overlapping calls on one GPU race).  In host code `scratch` is only a
// stand-in for the device copy: kernels get the address that
// hipGetSymbolAddress returns for the current device, never the name.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) __attribute__((used)) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[64];

// Device address of the current device's scratch copy (looked up once per
// device, with that device current).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(W4_E_UNSUPPORTED, "device %d: at most 64 devices", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return W4_OK;
}

}  // namespace

extern "C" {

int w4_abi_version(void) { return W4_ABI_VERSION; }
int w4_layout_version(void) { return W4_LAYOUT_VERSION; }

const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "W4_OK";
    case W4_E_NULL: return "W4_E_NULL: required pointer is NULL";
    case W4_E_SHAPE: return "W4_E_SHAPE: invalid size";
    case W4_E_DTYPE: return "W4_E_DTYPE: unsupported dtype combination";
    case W4_E_ALIGN: return "W4_E_ALIGN: pointer not 16-byte aligned";
    case W4_E_GROUP: return "W4_E_GROUP: unsupported group size";
    case W4_E_WORKSPACE: return "W4_E_WORKSPACE: workspace missing or too small";
    case W4_E_UNSUPPORTED: return "W4_E_UNSUPPORTED: not implemented for these arguments";
    case W4_E_HIP: return "W4_E_HIP: HIP runtime error";
    default: return "unknown w4_status";
  }
}

const char* w4_last_error(void) { return g_last_error.c_str(); }

size_t w4_prepack_B_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return (size_t)N * (size_t)K / 2u;
}

static int prepack_common(const void* w_in, void* w_packed, int64_t N, int64_t K, int operand, bool exllama,
                          void* stream) {
  if (!w_in || !w_packed) return fail(W4_E_NULL, "the input weight and w_packed are required");
  if (int st = check_shape(0, N, K)) return st;
  if ((N / 16) * (K / 128) >= ((int64_t)1 << 32))
    return fail(W4_E_SHAPE, "weights of 2^43 elements or more are not supported");
  if (operand != W4_OPERAND_I8 && operand != W4_OPERAND_F16)
    return fail(W4_E_DTYPE, "operand must be W4_OPERAND_I8 or W4_OPERAND_F16");
  if (!aligned(w_in, 16) || !aligned(w_packed, 16))
    return fail(W4_E_ALIGN, "the input weight and w_packed must be 16-byte aligned");
  const char* a = static_cast<const char*>(w_in);
  const char* b = static_cast<const char*>(w_packed);
  const size_t bytes = w4_prepack_B_bytes(N, K);
  if (a < b + bytes && b < a + bytes) return fail(W4_E_SHAPE, "input and output overlap");
  hipError_t e = launch_prepack(w_in, w_packed, N, K, operand, exllama, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prepack launch");
  return ok();
}

int w4_prepack_B(const void* w_logical, void* w_packed, int64_t N, int64_t K, int operand,
                 void* stream) {
  return prepack_common(w_logical, w_packed, N, K, operand, false, stream);
}

int w4_prepack_B_from_exllama(const void* w_words, void* w_packed, int64_t N, int64_t K, int operand,
                              void* stream) {
  return prepack_common(w_words, w_packed, N, K, operand, true, stream);
}

static int quant_common(const char* what, const void* x, int x_dtype, void* xq, int q_dtype, float* scales,
                        int64_t M, int64_t K, void* stream, bool per_tensor) {
  if (x_dtype != W4_F16 && x_dtype != W4_BF16) return fail(W4_E_DTYPE, "x_dtype must be W4_F16 or W4_BF16");
  if (q_dtype != W4_I8 && q_dtype != W4_FP8_E4M3)
    return fail(W4_E_DTYPE, "q_dtype must be W4_I8 or W4_FP8_E4M3");
  // a row is addressed with 32-bit buffer offsets: at most 2^29 elements
  if (M < 0 || K <= 0 || K % 8 || M > ((int64_t)1 << 31) - 1 || K > ((int64_t)1 << 29))
    return fail(W4_E_SHAPE, "need M >= 0, 0 < K <= 2^29, K %% 8 == 0 (M=%lld K=%lld)", (long long)M,
                (long long)K);
  if (M == 0) return ok();
  if (!x || !xq || !scales) return fail(W4_E_NULL, "x, xq and scales are required");
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(scales, 4))
    return fail(W4_E_ALIGN, "x and xq must be 16-byte aligned, scales 4-byte aligned");
  hipError_t e = per_tensor ? launch_quant_per_tensor(x, x_dtype, xq, q_dtype, scales, M, K, (hipStream_t)stream)
                            : launch_quant(x, x_dtype, xq, q_dtype, scales, M, K, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, what);
  return ok();
}

int w4_quant_act_per_token(const void* x, int x_dtype, void* xq, int q_dtype, float* scales,
                           int64_t M, int64_t K, void* stream) {
  return quant_common("quant launch", x, x_dtype, xq, q_dtype, scales, M, K, stream, false);
}

int w4_quant_act_per_tensor(const void* x, int x_dtype, void* xq, int q_dtype, float* scales,
                            int64_t M, int64_t K, void* stream) {
  return quant_common("per-tensor quant launch", x, x_dtype, xq, q_dtype, scales, M, K, stream, true);
}

int w4_rmsnorm_quant_per_token(const void* x, int x_dtype, const void* gamma, float eps, void* xq, int q_dtype,
                               float* scales, int64_t M, int64_t K, void* stream) {
  if (x_dtype != W4_F16 && x_dtype != W4_BF16) return fail(W4_E_DTYPE, "x_dtype must be W4_F16 or W4_BF16");
  if (q_dtype != W4_I8 && q_dtype != W4_FP8_E4M3)
    return fail(W4_E_DTYPE, "q_dtype must be W4_I8 or W4_FP8_E4M3");
  if (M < 0 || K <= 0 || K % 8 || M > ((int64_t)1 << 31) - 1 || K > ((int64_t)1 << 29))
    return fail(W4_E_SHAPE, "need M >= 0, 0 < K <= 2^29, K %% 8 == 0 (M=%lld K=%lld)", (long long)M,
                (long long)K);
  if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(W4_E_SHAPE, "eps must be positive and finite");
  if (M == 0) return ok();
  if (!x || !gamma || !xq || !scales) return fail(W4_E_NULL, "x, gamma, xq and scales are required");
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(xq, 16) || !aligned(scales, 4))
    return fail(W4_E_ALIGN, "x, gamma and xq must be 16-byte aligned, scales 4-byte aligned");
  hipError_t e = launch_rmsnorm_quant(x, x_dtype, gamma, eps, xq, q_dtype, scales, M, K,
                                     (int)g_norm_exact_sum.load(), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rmsnorm-quant launch");
  return ok();
}

size_t w4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group_size, int a_dtype) {
  const int op = op_of(a_dtype);
  const bool w4a16 = op == OP_F16 || op == OP_BF16;
  if (op < 0 || check_shape(M, N, K) || check_group(group_size, K, w4a16)) return 0;
  GemmPlan plan;
  const bool grouped = resolve_group(group_size, K) != K;
  if (make_plan(M, N, K, grouped, op, &plan, false, subgroups(group_size, K))) return 0;
  size_t need = workspace_for(plan, M, N);
  // int8: also large enough for the asymmetric GEMM (w4a8_gemm_zp), whose
  // plan may differ
  GemmPlan zp_plan;
  if (op == OP_I8 && make_plan(M, N, K, grouped, op, &zp_plan, true) == W4_OK) {
    const size_t zneed = workspace_for(zp_plan, M, N);
    if (zneed > need) need = zneed;
  }
  return need;
}

int w4_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t group_size, int a_dtype, int* path, int* splitk,
                 int* tile_m, int* tile_n) {
  const int op = op_of(a_dtype);
  if (op < 0) return fail(W4_E_DTYPE, "unknown a_dtype");
  if (int st = check_shape(M, N, K)) return st;
  if (int st = check_group(group_size, K, op == OP_F16 || op == OP_BF16)) return st;
  GemmPlan plan;
  if (int st = make_plan(M, N, K, resolve_group(group_size, K) != K, op, &plan, false, subgroups(group_size, K)))
    return st;
  if (path) *path = plan.path;
  if (splitk) *splitk = plan.splitk;
  if (tile_m) *tile_m = plan.path == PATH_SKINNY ? 16 : plan.bm;
  if (tile_n) *tile_n = plan.bn;
  return ok();
}

static int validate_w4a8(const void* aq, int a_dtype, const void* b_packed, int wtype, int64_t group_size,
                         int64_t M, int64_t N, int64_t K) {
  if (a_dtype != W4_I8 && a_dtype != W4_FP8_E4M3)
    return fail(W4_E_DTYPE, "a_dtype must be W4_I8 or W4_FP8_E4M3");
  if (wtype != W4_INT4 && wtype != W4_UINT4B8)
    return fail(W4_E_DTYPE, "W4A8 weights are W4_INT4 or W4_UINT4B8 (symmetric)");
  if (int st = check_shape(M, N, K)) return st;
  if (int st = check_group(group_size, K)) return st;
  if (a_dtype == W4_I8 && resolve_group(group_size, K) == K && K > 131072)
    return fail(W4_E_SHAPE, "int8 per-channel accumulation needs K <= 131072 (int32 range)");
  if (!b_packed || (M > 0 && !aq)) return fail(W4_E_NULL, "aq and b_packed are required");
  if (!aligned(aq, 16) || !aligned(b_packed, 16)) return fail(W4_E_ALIGN, "aq and b_packed must be 16-byte aligned");
  return W4_OK;
}

// Every check of w4a8_gemm but the workspace's.
static int validate_w4a8_gemm(const void* aq, int a_dtype, const float* a_scales, const void* b_packed, int wtype,
                              const void* b_scales, int s_dtype, int64_t group_size, const void* bias,
                              const void* out, int out_dtype, int64_t M, int64_t N, int64_t K) {
  if (int st = validate_w4a8(aq, a_dtype, b_packed, wtype, group_size, M, N, K)) return st;
  if (s_dtype != W4_F32 && s_dtype != W4_F16 && s_dtype != W4_BF16)
    return fail(W4_E_DTYPE, "s_dtype must be W4_F32, W4_F16 or W4_BF16");
  if (out_dtype != W4_F16 && out_dtype != W4_BF16) return fail(W4_E_DTYPE, "out_dtype must be W4_F16 or W4_BF16");
  if (!b_scales || (M > 0 && (!a_scales || !out))) return fail(W4_E_NULL, "a_scales, b_scales and out are required");
  if (!aligned(out, 16) || !aligned(a_scales, 4) || !aligned(b_scales, s_dtype == W4_F32 ? 4 : 2) ||
      !aligned(bias, 2))
    return fail(W4_E_ALIGN, "out must be 16-byte aligned; scales and bias naturally aligned");
  return W4_OK;
}

int w4a8_gemm(const void* aq, int a_dtype, const float* a_scales, const void* b_packed, int wtype,
              const void* b_scales, int s_dtype, int64_t group_size, const void* bias, void* out,
              int out_dtype, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
              void* stream) {
  if (int st = validate_w4a8_gemm(aq, a_dtype, a_scales, b_packed, wtype, b_scales, s_dtype, group_size, bias, out,
                                  out_dtype, M, N, K))
    return st;
  const int64_t g = resolve_group(group_size, K);
  GemmArgs args{};
  args.a = aq;
  args.a_scales = a_scales;
  args.b = static_cast<const uint32_t*>(b_packed);
  args.s = b_scales;
  args.bias = bias;
  args.out = out;
  args.M = M;
  args.N = N;
  args.K = K;
  args.G = (int)(K / g);
  args.s_dtype = s_dtype;
  args.out_dtype = out_dtype;
  args.z_dtype = W4_F16;
  args.mode = MODE_OUTPUT;
  return run_gemm(args, op_of(a_dtype), g != K, wtype == W4_UINT4B8, workspace, workspace_bytes, stream);
}

int w4a8_gemm_no_alloc(const void* aq, int a_dtype, const float* a_scales, const void* b_packed, int wtype,
                       const void* b_scales, int s_dtype, int64_t group_size, const void* bias, void* out,
                       int out_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  // the checks of w4a8_gemm first, so that an invalid call reports the same error
  if (int st = validate_w4a8_gemm(aq, a_dtype, a_scales, b_packed, wtype, b_scales, s_dtype, group_size, bias, out,
                                  out_dtype, M, N, K))
    return st;
  const size_t need = w4_gemm_workspace_bytes(M, N, K, group_size, a_dtype);
  if (need > kScratchBytes)
    return fail(W4_E_WORKSPACE,
                "w4a8_gemm_no_alloc: this problem's split-K workspace (%zu bytes) exceeds the built-in %zu; "
                "call w4a8_gemm with a workspace", need, kScratchBytes);
  void* ws = nullptr;
  if (need) {
    if (int st = scratch_address(&ws)) return st;
  }
  return w4a8_gemm(aq, a_dtype, a_scales, b_packed, wtype, b_scales, s_dtype, group_size, bias, out, out_dtype, M,
                   N, K, ws, need ? kScratchBytes : 0, stream);
}

int w4a8_gemm_quant_fused(const void* x, int x_dtype, int q_dtype, const void* b_packed, int wtype,
                          const void* b_scales, int s_dtype, int64_t group_size, const void* bias, void* out,
                          int out_dtype, int64_t M, int64_t N, int64_t K, float* a_scales_out, void* stream) {
  if (x_dtype != W4_F16 && x_dtype != W4_BF16) return fail(W4_E_DTYPE, "x_dtype must be W4_F16 or W4_BF16");
  if (q_dtype != W4_I8 && q_dtype != W4_FP8_E4M3) return fail(W4_E_DTYPE, "q_dtype must be W4_I8 or W4_FP8_E4M3");
  if (int st = validate_w4a8(x, q_dtype, b_packed, wtype, group_size, M, N, K)) return st;
  if (s_dtype != W4_F32 && s_dtype != W4_F16 && s_dtype != W4_BF16)
    return fail(W4_E_DTYPE, "s_dtype must be W4_F32, W4_F16 or W4_BF16");
  if (out_dtype != W4_F16 && out_dtype != W4_BF16) return fail(W4_E_DTYPE, "out_dtype must be W4_F16 or W4_BF16");
  if (!b_scales || (M > 0 && !out)) return fail(W4_E_NULL, "b_scales and out are required");
  if (!aligned(out, 16) || !aligned(b_scales, s_dtype == W4_F32 ? 4 : 2) || !aligned(bias, 2) ||
      !aligned(a_scales_out, 4))
    return fail(W4_E_ALIGN, "out must be 16-byte aligned; scales and bias naturally aligned");
  if (M == 0) return ok();
  const int64_t g = resolve_group(group_size, K);
  const bool grouped = g != K;
  const int op = op_of(q_dtype);
  GemmPlan plan;
  if (int st = make_plan(M, N, K, grouped, op, &plan)) return st;
  const int ns = plan.bn / 16;
  // the codes stay in the small-M kernel's LDS next to its tables
  const int64_t lds = skinny_table_bytes(op, grouped, K / g, ns) + M * K + 32 + skinny_static_lds(op, grouped, ns);
  if (plan.path != PATH_SKINNY || lds > 65536)
    return fail(W4_E_UNSUPPORTED,
                "fused quantisation needs the small-M kernel with M*K codes in LDS (M=%lld K=%lld): "
                "use w4_quant_act_per_token and w4a8_gemm", (long long)M, (long long)K);
  GemmArgs args{};
  args.x = x;
  args.x_dtype = x_dtype;
  args.a_scales_out = a_scales_out;
  args.b = static_cast<const uint32_t*>(b_packed);
  args.s = b_scales;
  args.bias = bias;
  args.out = out;
  args.M = M;
  args.N = N;
  args.K = K;
  args.G = (int)(K / g);
  args.s_dtype = s_dtype;
  args.out_dtype = out_dtype;
  args.z_dtype = W4_F16;
  args.mode = MODE_OUTPUT;
  hipError_t e = launch_gemm(args, op, grouped, wtype == W4_UINT4B8, false, plan, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fused GEMM launch");
  return ok();
}

int w4a8_gemm_zp(const void* aq, const float* a_scales, const void* b_packed, const void* b_scales, int s_dtype,
                 const void* zeros, int z_dtype, int64_t group_size, const void* bias, void* out, int out_dtype,
                 int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = validate_w4a8(aq, W4_I8, b_packed, W4_UINT4B8, group_size, M, N, K)) return st;
  if (s_dtype != W4_F32 && s_dtype != W4_F16 && s_dtype != W4_BF16)
    return fail(W4_E_DTYPE, "s_dtype must be W4_F32, W4_F16 or W4_BF16");
  if (z_dtype != W4_F32 && z_dtype != W4_F16 && z_dtype != W4_BF16)
    return fail(W4_E_DTYPE, "z_dtype must be W4_F32, W4_F16 or W4_BF16");
  if (out_dtype != W4_F16 && out_dtype != W4_BF16) return fail(W4_E_DTYPE, "out_dtype must be W4_F16 or W4_BF16");
  const int64_t g = resolve_group(group_size, K);
  // 16 sum(a (u - z)) in int32 over a whole-K group: |.| <= 16 * 127 * 15 * K
  if (g == K && K > 65536) return fail(W4_E_SHAPE, "per-channel zero-points need K <= 65536 (int32 range)");
  if (!b_scales || !zeros || (M > 0 && (!a_scales || !out)))
    return fail(W4_E_NULL, "a_scales, b_scales, zeros and out are required");
  if (!aligned(out, 16) || !aligned(a_scales, 4) || !aligned(b_scales, s_dtype == W4_F32 ? 4 : 2) ||
      !aligned(zeros, z_dtype == W4_F32 ? 4 : 2) || !aligned(bias, 2))
    return fail(W4_E_ALIGN, "out must be 16-byte aligned; scales, zeros and bias naturally aligned");
  GemmArgs args{};
  args.a = aq;
  args.a_scales = a_scales;
  args.b = static_cast<const uint32_t*>(b_packed);
  args.s = b_scales;
  args.z = zeros;
  args.bias = bias;
  args.out = out;
  args.M = M;
  args.N = N;
  args.K = K;
  args.G = (int)(K / g);
  args.s_dtype = s_dtype;
  args.out_dtype = out_dtype;
  args.z_dtype = z_dtype;
  args.mode = MODE_OUTPUT;
  // raw uint4 codes: the int8 operand holds 16 (u - 8), the kernels subtract (z - 8) sum(a)
  return run_gemm(args, OP_I8, g != K, true, workspace, workspace_bytes, stream, true);
}

static int validate_w4a16(const void* a, int a_dtype, const void* b_packed, int wtype, const void* zeros,
                          int64_t group_size, int64_t M, int64_t N, int64_t K) {
  if (a_dtype != W4_F16 && a_dtype != W4_BF16) return fail(W4_E_DTYPE, "a_dtype must be W4_F16 or W4_BF16");
  if (wtype != W4_UINT4 && wtype != W4_UINT4B8)
    return fail(W4_E_DTYPE, "W4A16 weights are W4_UINT4 or W4_UINT4B8");
  if (wtype == W4_UINT4B8 && zeros) return fail(W4_E_DTYPE, "W4_UINT4B8 weights take no zero-points");
  if (int st = check_shape(M, N, K)) return st;
  if (int st = check_group(group_size, K, true)) return st;
  if (!b_packed || (M > 0 && !a)) return fail(W4_E_NULL, "a and b_packed are required");
  if (!aligned(a, 16) || !aligned(b_packed, 16)) return fail(W4_E_ALIGN, "a and b_packed must be 16-byte aligned");
  if (!aligned(zeros, 2)) return fail(W4_E_ALIGN, "zeros must be 2-byte aligned");
  return W4_OK;
}

int w4a16_gemm(const void* a, int a_dtype, const void* b_packed, int wtype, const void* scales,
               const void* zeros, int64_t group_size, const void* bias, void* out, int64_t M, int64_t N,
               int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = validate_w4a16(a, a_dtype, b_packed, wtype, zeros, group_size, M, N, K)) return st;
  if (!scales || (M > 0 && !out)) return fail(W4_E_NULL, "scales and out are required");
  if (!aligned(out, 16) || !aligned(scales, 2) || !aligned(bias, 2))
    return fail(W4_E_ALIGN, "out must be 16-byte aligned; scales and bias 2-byte aligned");
  const int64_t g = resolve_group(group_size, K);
  GemmArgs args{};
  args.a = a;
  args.b = static_cast<const uint32_t*>(b_packed);
  args.s = scales;
  args.z = zeros;
  args.bias = bias;
  args.out = out;
  args.M = M;
  args.N = N;
  args.K = K;
  args.G = (int)(K / g);
  args.s_dtype = a_dtype;
  args.out_dtype = a_dtype;
  args.z_dtype = a_dtype;
  args.mode = MODE_OUTPUT;
  return run_gemm(args, op_of(a_dtype), g != K, false, workspace, workspace_bytes, stream);
}

int w4a16_gemm_prescaled_zeros(const void* a, int a_dtype, const void* b_packed, const void* scales,
                               const void* zeros_scaled, int64_t group_size, const void* bias, void* out, int64_t M,
                               int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = validate_w4a16(a, a_dtype, b_packed, W4_UINT4, zeros_scaled, group_size, M, N, K)) return st;
  if (resolve_group(group_size, K) != 128 || K == 128)
    return fail(W4_E_GROUP, "pre-scaled zero-points take groups of 128 (group_size=%lld)", (long long)group_size);
  if (!scales || !zeros_scaled || (M > 0 && !out)) return fail(W4_E_NULL, "scales, zeros_scaled and out are required");
  if (!aligned(out, 16) || !aligned(scales, 2) || !aligned(bias, 2))
    return fail(W4_E_ALIGN, "out must be 16-byte aligned; scales and bias 2-byte aligned");
  GemmArgs args{};
  args.a = a;
  args.b = static_cast<const uint32_t*>(b_packed);
  args.s = scales;
  args.z = zeros_scaled;
  args.bias = bias;
  args.out = out;
  args.M = M;
  args.N = N;
  args.K = K;
  args.G = (int)(K / 128);
  args.s_dtype = a_dtype;
  args.out_dtype = a_dtype;
  args.z_dtype = a_dtype;
  args.prescaled_zeros = true;
  args.mode = MODE_OUTPUT;
  return run_gemm(args, op_of(a_dtype), true, false, workspace, workspace_bytes, stream);
}

static int check_window(int64_t M, int64_t N, int64_t m0, int64_t m1, int64_t n0, int64_t n1) {
  if (m0 < 0 || m0 > m1 || m1 > M || n0 < 0 || n0 > n1 || n1 > N)
    return fail(W4_E_SHAPE, "window rows [%lld,%lld) cols [%lld,%lld) outside [0,%lld) x [0,%lld)",
                (long long)m0, (long long)m1, (long long)n0, (long long)n1, (long long)M, (long long)N);
  return W4_OK;
}

int w4a8_gemm_partials(const void* aq, int a_dtype, const void* b_packed, int wtype, int64_t group_size,
                       int64_t M, int64_t N, int64_t K, int64_t m0, int64_t m1, int64_t n0, int64_t n1,
                       void* partials, void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = validate_w4a8(aq, a_dtype, b_packed, wtype, group_size, M, N, K)) return st;
  if (int st = check_window(M, N, m0, m1, n0, n1)) return st;
  if (m1 > m0 && n1 > n0 && !partials) return fail(W4_E_NULL, "partials is required");
  if (!aligned(partials, 4)) return fail(W4_E_ALIGN, "partials must be 4-byte aligned");
  const int64_t g = resolve_group(group_size, K);
  GemmArgs args{};
  args.a = aq;
  args.b = static_cast<const uint32_t*>(b_packed);
  args.partials = partials;
  args.M = M;
  args.N = N;
  args.K = K;
  args.G = (int)(K / g);
  args.s_dtype = W4_F32;
  args.out_dtype = W4_F16;
  args.mode = MODE_PARTIALS;
  args.m0 = m0;
  args.m1 = m1;
  args.n0 = n0;
  args.n1 = n1;
  return run_gemm(args, op_of(a_dtype), g != K, wtype == W4_UINT4B8, workspace, workspace_bytes, stream);
}

int w4a16_gemm_partials(const void* a, int a_dtype, const void* b_packed, int wtype, const void* zeros,
                        int64_t group_size, int64_t M, int64_t N, int64_t K, int64_t m0, int64_t m1,
                        int64_t n0, int64_t n1, void* partials, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (int st = validate_w4a16(a, a_dtype, b_packed, wtype, zeros, group_size, M, N, K)) return st;
  if (int st = check_window(M, N, m0, m1, n0, n1)) return st;
  if (m1 > m0 && n1 > n0 && !partials) return fail(W4_E_NULL, "partials is required");
  if (!aligned(partials, 4)) return fail(W4_E_ALIGN, "partials must be 4-byte aligned");
  const int64_t g = resolve_group(group_size, K);
  GemmArgs args{};
  args.a = a;
  args.b = static_cast<const uint32_t*>(b_packed);
  args.z = zeros;
  args.partials = partials;
  args.M = M;
  args.N = N;
  args.K = K;
  args.G = (int)(K / g);
  args.s_dtype = a_dtype;
  args.out_dtype = a_dtype;
  args.z_dtype = a_dtype;
  args.mode = MODE_PARTIALS;
  args.m0 = m0;
  args.m1 = m1;
  args.n0 = n0;
  args.n1 = n1;
  return run_gemm(args, op_of(a_dtype), g != K, false, workspace, workspace_bytes, stream);
}

int w4_set_option(const char* key, int64_t value) {
  if (!key) return fail(W4_E_NULL, "key is required");
  if (!strcmp(key, "force_path")) {
    if (value < 0 || value > 4) return fail(W4_E_SHAPE, "force_path must be 0, 1, 2, 3 or 4");
    g_force_path.store(value);
    return ok();
  }
  if (!strcmp(key, "splitk")) {
    if (value < 0 || value > 64) return fail(W4_E_SHAPE, "splitk must be in [0, 64]");
    g_splitk.store(value);
    return ok();
  }
  if (!strcmp(key, "skinny_strips")) {
    if (value < 0 || value > 4 || value == 3) return fail(W4_E_SHAPE, "skinny_strips must be 0, 1, 2 or 4");
    g_skinny_strips.store(value);
    return ok();
  }
  if (!strcmp(key, "tiled_bm")) {
    if (value != 0 && value != 32 && value != 64 && value != 128 && value != 256)
      return fail(W4_E_SHAPE, "tiled_bm must be 0, 32, 64, 128 or 256");
    g_tiled_bm.store(value);
    return ok();
  }
  if (!strcmp(key, "norm_exact_sum")) {
    if (value != 0 && value != 1) return fail(W4_E_SHAPE, "norm_exact_sum must be 0 or 1");
    g_norm_exact_sum.store(value);
    return ok();
  }
  if (!strcmp(key, "schedule_table")) {
    if (value != 0 && value != 1) return fail(W4_E_SHAPE, "schedule_table must be 0 or 1");
    g_schedule_table.store(value);
    return ok();
  }
  return fail(W4_E_UNSUPPORTED, "unknown option '%s'", key);
}

int64_t w4_get_option(const char* key) {
  if (!key) return -1;
  if (!strcmp(key, "force_path")) return g_force_path.load();
  if (!strcmp(key, "splitk")) return g_splitk.load();
  if (!strcmp(key, "skinny_strips")) return g_skinny_strips.load();
  if (!strcmp(key, "tiled_bm")) return g_tiled_bm.load();
  if (!strcmp(key, "norm_exact_sum")) return g_norm_exact_sum.load();
  if (!strcmp(key, "schedule_table")) return g_schedule_table.load();
  return -1;
}

int w4_schedule_add(int a_dtype, int group_mode, int64_t N, int64_t K, int64_t m_lo, int64_t m_hi, int path,
                    int splitk, int tile_m, int strips) {
  if (op_of(a_dtype) < 0) return fail(W4_E_DTYPE, "unknown a_dtype");
  if (group_mode != 0 && group_mode != 1) return fail(W4_E_SHAPE, "group_mode must be 0 or 1");
  if (N <= 0 || K <= 0 || m_lo < 0 || m_hi < m_lo)
    return fail(W4_E_SHAPE, "need N > 0, K > 0, 0 <= m_lo <= m_hi");
  if (path < 0 || path > 4) return fail(W4_E_SHAPE, "path must be 0, 1, 2, 3 or 4");
  if (splitk < 0 || splitk > 64) return fail(W4_E_SHAPE, "splitk must be in [0, 64]");
  if (tile_m != 0 && tile_m != 32 && tile_m != 64 && tile_m != 128 && tile_m != 256)
    return fail(W4_E_SHAPE, "tile_m must be 0, 32, 64, 128 or 256");
  if (strips < 0 || strips > 4 || strips == 3) return fail(W4_E_SHAPE, "strips must be 0, 1, 2 or 4");
  if (path == 1 && m_hi > 16) return fail(W4_E_SHAPE, "the small-M kernel handles M <= 16");
  std::lock_guard<std::mutex> lock(g_sched_mutex);
  // a later entry for the same problems replaces an earlier one
  g_sched_user.insert(g_sched_user.begin(),
                      SchedEntry{a_dtype, group_mode, N, K, m_lo, m_hi, path, splitk, tile_m, strips});
  return ok();
}

int w4_schedule_clear(void) {
  std::lock_guard<std::mutex> lock(g_sched_mutex);
  g_sched_user.clear();
  return ok();
}

}  // extern "C"
