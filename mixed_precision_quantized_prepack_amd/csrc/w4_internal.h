// Internal interface between the C ABI (w4_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

// Matrix-core operand class of a GEMM (the activation type it multiplies).
enum Op : int { OP_I8 = 0, OP_FP8 = 1, OP_F16 = 2, OP_BF16 = 3 };

enum Path : int { PATH_AUTO = 0, PATH_SKINNY = 1, PATH_TILED = 2, PATH_STREAM = 3, PATH_PINGPONG = 4 };
enum Mode : int { MODE_OUTPUT = 0, MODE_PARTIALS = 1 };

// Everything a GEMM kernel reads, in element units unless noted.
struct GemmArgs {
  const void* a;           // [M][K] activations: int8 / e4m3 bytes, or fp16 / bf16
  const float* a_scales;   // [M] per-token scales (W4A8) or nullptr (W4A16)
  const uint32_t* b;       // PB-v1 words
  const void* s;           // weight scales: [N] (per channel) or [N][G]
  const void* z;           // zero-points [N][G] (W4A16, asymmetric W4A8) or nullptr (z = 8)
  const void* bias;        // [N] in out dtype, or nullptr
  void* out;               // [M][N]
  void* ws;                // split-K slots [splitk][M][N] of 4-byte values
  void* partials;          // MODE_PARTIALS: [G][m1-m0][n1-n0]
  int64_t M, N, K;
  int G;                   // K / group_size
  int s_dtype;             // W4_F32 / W4_F16 / W4_BF16
  int out_dtype;           // W4_F16 / W4_BF16
  int z_dtype;             // zero-point storage: W4_F16 / W4_BF16 / W4_F32
  // fused per-token quantisation (small-M kernel): x holds the fp16 / bf16
  // activations [M][K] (a is unused); the per-token scales go to
  // a_scales_out when it is not null
  const void* x;
  int x_dtype;
  float* a_scales_out;
  // W4A16 with pre-scaled zero-points: z holds zs (in the activation dtype),
  // subtracted after the scale
  bool prescaled_zeros;
  int mode;                // Mode
  int64_t m0, m1, n0, n1;  // partials window
};

// Largest workgroup of the small-M kernel, in waves (each wave takes every
// S-th K block of the workgroup's strips).  Ungrouped 8-bit problems fit in
// 128 registers per lane and may use 16 waves; the others keep more state
// per wave and are limited to 8.
constexpr int skinny_max_waves(int op, bool grouped) {
  return (op == OP_I8 || op == OP_FP8) && !grouped ? 16 : 8;
}

// LDS tables of the small-M kernel (grouped problems only): group scales,
// and for W4A16 the zero-point terms, each [strips][groups][16] fp32
// followed by a 16-float pad.
// (asymmetric int8 W4A8 also keeps a zero-point table).
constexpr int skinny_tables(int op, bool grouped, bool zp = false) {
  return grouped ? ((op == OP_BF16 || op == OP_F16 || zp) ? 2 : 1) : 0;
}
inline int64_t skinny_table_bytes(int op, bool grouped, int64_t groups, int strips, bool zp = false) {
  return (int64_t)skinny_tables(op, grouped, zp) * (strips * groups * 16 + 16) * 4;
}
// Largest table the small-M kernel stages; larger problems use the tiled kernel.
constexpr int64_t kSkinnyTableMax = 48 * 1024;

struct GemmPlan {
  int path;    // PATH_SKINNY, PATH_TILED, PATH_STREAM or PATH_PINGPONG
  int splitk;  // skinny: waves per workgroup splitting K; tiled: K splits across workgroups
  int bm, bn;  // tiled block tile (rows of A, columns of W)
};

// Block tile of the tiled kernel for an operand class / grouping.
void tiled_tile(int op, bool grouped, int tall, int* bm, int* bn, bool zp = false);

hipError_t launch_prepack(const void* w_in, void* w_packed, int64_t N, int64_t K, int operand, bool exllama,
                          hipStream_t stream);
hipError_t launch_quant(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                        int64_t K, hipStream_t stream);
hipError_t launch_quant_per_tensor(const void* x, int x_dtype, void* xq, int q_dtype, float* scales, int64_t M,
                                   int64_t K, hipStream_t stream);
hipError_t launch_rmsnorm_quant(const void* x, int x_dtype, const void* gamma, float eps, void* xq, int q_dtype,
                                float* scales, int64_t M, int64_t K, int exact_sum, hipStream_t stream);
// Bytes of LDS the small-M kernel declares statically (its wave-order
// reduction buffer and the fused quantiser's row maxima and scales).
constexpr int64_t skinny_static_lds(int op, bool grouped, int strips) {
  return (int64_t)skinny_max_waves(op, grouped) * strips * 64 * 4 * 4 + 2 * 16 * 4;
}

// zp: asymmetric int8 W4A8 (op OP_I8, flip set: raw uint4 codes, zero-points in args.z).
// The fused quantisation (args.x set) takes the small-M kernel (plan.path == PATH_SKINNY).
hipError_t launch_gemm(const GemmArgs& args, int op, bool grouped, bool flip, bool zp, const GemmPlan& plan,
                       hipStream_t stream);

// The streaming kernel (8-bit operands, symmetric weights; plan.path ==
// PATH_STREAM): tiles 32 x 256, 64 x 256 and 128 x 128.
// Ping-pong kernel (int8 per channel, symmetric weights; plan.bm = 256 or 128
// rows, plan.bn = 256 columns).
hipError_t launch_pingpong(const GemmArgs& args, bool flip, const GemmPlan& plan, hipStream_t stream);
hipError_t launch_stream(const GemmArgs& args, int op, bool grouped, bool flip, const GemmPlan& plan,
                         hipStream_t stream);
// Steps the streaming kernel's LDS ring holds for a tile of 16 mt rows and 4 nt
// n-blocks: as many 128-deep steps (activation tile + the four waves' weight
// blocks) as fit 120 KiB, at most 8; 32 KiB more hold a grouped problem's
// scale table.
constexpr int stream_stages(int mt, int nt) {
  return (120 * 1024) / (mt * 16 * 128 + 4 * nt * 1024) > 8 ? 8 : (120 * 1024) / (mt * 16 * 128 + 4 * nt * 1024);
}
// Groups of 128 the streaming kernel's 32 KiB scale table holds for a tile of
// bn columns (the K range of one split).
constexpr int stream_table_groups(int bn) { return 8192 / bn; }
// Sum of the split-K slots and the epilogue (the workspace of a split plan).
hipError_t launch_splitk_reduce(const GemmArgs& args, int op, bool grouped, int splitk, hipStream_t stream);

}  // namespace w4
