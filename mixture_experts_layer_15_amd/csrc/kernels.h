// kernels.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/moe.h).  Every launcher only
// enqueues on the given stream and returns the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

// Top-k routing parameters: k slots per token, softmax temperature tau, gates
// renormalised over the chosen experts or not; theta > 0 makes the count per
// token dynamic (the fewest of the k ranked experts, at least k_min, whose
// softmax mass reaches theta; the slots past it hold expert -1, gate 0).
struct TopkParams {
    int k;
    float tau;
    int renorm;
    int k_min;
    float theta;
};

// Router: logits = x W_r + b (fp32 accumulation), softmax(l / tau), top-k, gates.
hipError_t launch_route(int dtype, const void* x, const void* w_router, const float* bias,
                        float* logits, int32_t* idx, float* gate, long long T, int d, int E,
                        TopkParams tp, hipStream_t s);
// Top-k and gates from given fp32 logits.
hipError_t launch_route_from_logits(const float* logits, int32_t* idx, float* gate,
                                    long long T, int E, TopkParams tp, hipStream_t s);

// Dispatch.  Tokens are cut into nblk blocks of blk_tokens (a multiple of 256)
// with nblk <= 256; workspace holds two [nblk][E] int32 tables.
// The kernels walk "tokens" of k choices each.  In token order those are the
// real tokens; in choice order they are the T*k single choices in (choice,
// token) order (T = Tr * kr, k = 1), mapped back to the real slots.
struct DispatchPlan {
    long long T;           // tokens the kernels walk
    int E, k;              // experts; choices per walked token
    long long C;
    int blk_tokens, nblk;
    long long Tr;          // real tokens
    int kr;                // real choices per token
    bool choice_order;
    bool padded;           // padded layout: expert e owns rows e*C .. e*C + C - 1
    // dynamic expert counts: C is taken on the device from the realised
    // assignments, ceil(cap_num A / (cap_den E)) (C above is then only the
    // host's upper bound)
    bool dyn;
    int cap_num, cap_den;
};
DispatchPlan plan_dispatch(long long T, int E, int k, long long C, int policy = 0,
                           int layout = 0, bool dyn = false, int cap_num = 0, int cap_den = 0);
size_t dispatch_workspace_bytes(const DispatchPlan& p);
// scatter = false leaves x_perm unwritten (for a consumer that gathers rows of
// x through token_of_row itself).  In the padded layout the empty rows get
// token_of_row -1 and (with scatter) zero rows in x_perm.
hipError_t launch_dispatch(const DispatchPlan& p, int dtype, const int32_t* idx, const void* x,
                           void* x_perm, int32_t* count, int32_t* offset, int32_t* row_of,
                           int32_t* token_of_row, void* workspace, int d, hipStream_t s,
                           bool scatter = true);

// x_perm[row_of[t][j]] = x[t] for every kept (t, j) (rows of row_bytes bytes).
// Padded layout: zero the rows of buf [E * C][row_bytes] that hold no token
// (and mark them -1 in token_of_row, as the dispatch does).
hipError_t launch_zero_empty_rows(const int32_t* count, long long C, int E, int32_t* token_of_row,
                                  void* buf, int row_bytes, hipStream_t s);
hipError_t launch_scatter_rows(const void* x, const int32_t* row_of, void* x_perm, long long T,
                               int row_bytes, int k, hipStream_t s);

// Load-balance PID controller step (see moe_pid_update); E <= 256.
hipError_t launch_pid_update(const int32_t* count, int E, double kp, double ki, double kd,
                             double scale, double* state, float* bias, hipStream_t s);
// Expert-load telemetry (8 fp64 values, see moe_load_stats).
hipError_t launch_load_stats(const int32_t* count, int E, long long C, double* stats,
                             hipStream_t s, bool dyn = false, int cap_num = 0, int cap_den = 0,
                             long long T = 0);

// Grouped GeGLU expert FFN (gate/up GEMM with fused epilogue, then down GEMM).
hipError_t launch_expert_ffn(int dtype, const void* x_perm, const int32_t* off,
                             const void* w_gate, const void* w_up, const void* w_down,
                             void* h, void* y_perm, int E, int d, int d_ff,
                             long long max_rows, int grid_cap, hipStream_t s);

// The two halves of the expert FFN, one launch each.
hipError_t launch_gate_up(int dtype, const void* x_perm, const int32_t* off, const void* w_gate,
                          const void* w_up, void* h, int E, int d, int d_ff, long long max_rows,
                          int grid_cap, hipStream_t s, const int32_t* gather_rows = nullptr);
// With y != nullptr (bf16, top-1, every token kept) the down GEMM writes the
// layer output y[token_of_row[r]] = gate * O[r] itself instead of y_perm,
// bit-identical to launch_combine over y_perm.
hipError_t launch_down(int dtype, const void* h, const int32_t* off, const void* w_down,
                       void* y_perm, int E, int d, int d_ff, long long max_rows, int grid_cap,
                       hipStream_t s, const float* gate = nullptr,
                       const int32_t* token_of_row = nullptr, void* y = nullptr);

// bf16 MFMA kernels (gemm_mfma.hip); cus = workgroups of the persistent grid.
// gate/up reads its rows from a: x_perm (a_rows == nullptr), or x gathered
// through a_rows = token_of_row.
hipError_t launch_mfma_gate_up(const uint16_t* a, const int32_t* a_rows, const int32_t* off,
                               const uint16_t* w_gate,
                               const uint16_t* w_up, uint16_t* h, int E, int d, int d_ff,
                               long long max_rows, int cus, hipStream_t s);
hipError_t launch_mfma_down(const uint16_t* h, const int32_t* off, const uint16_t* w_down,
                            uint16_t* y_perm, int E, int d, int d_ff, long long max_rows,
                            int cus, hipStream_t s, const float* gate = nullptr,
                            const int32_t* tor = nullptr, uint16_t* y = nullptr);

// The down GEMM in two K slices (bf16 in, fp32 partials P[2][rows][d] out,
// p_stride floats apart), for layers where down_split_applies(): small
// experts whose 320 x 256 down tiles alone would leave CUs idle.
bool down_split_applies(long long max_rows, int E, int d, int d_ff, int cus);
hipError_t launch_mfma_down_split(const uint16_t* h, const int32_t* off, const uint16_t* w_down,
                                  float* P, long long p_stride, int E, int d, int d_ff,
                                  long long max_rows, int cus, hipStream_t s);
// y[t] = gate[t] * bf16(P[0][r] + P[1][r]) with r = row_of[t], for top-1
// layers that keep every token (bf16 out, rounded as the combine rounds).
hipError_t launch_combine_split(const float* P, long long p_stride, const int32_t* row_of,
                                const float* gate, void* y, long long T, int d, hipStream_t s);

// The gate/up GEMM's two products stored separately (bf16): g = X W_gate,
// u = X W_up (rows of X as in launch_mfma_gate_up).
hipError_t launch_mfma_gate_up_pre(const uint16_t* a, const int32_t* a_rows, const int32_t* off,
                                   const uint16_t* w_gate, const uint16_t* w_up, uint16_t* g,
                                   uint16_t* u, int E, int d, int d_ff, long long max_rows,
                                   int cus, hipStream_t s);

// Plain grouped GEMM C[rows][N] = A[rows][K] B[e] (bf16 out), A's rows read
// directly (a_rows == nullptr) or gathered through a_rows (gemm_mfma.hip).
hipError_t launch_mfma_grouped(const uint16_t* A, const int32_t* a_rows, const int32_t* off,
                               const uint16_t* B, uint16_t* C, int E, int K, int N,
                               long long max_rows, int cus, hipStream_t s,
                               const float* gate = nullptr, const int32_t* tor = nullptr,
                               uint16_t* y = nullptr);

// Dense bf16 GEMM with optional bias and GELU epilogue (gemm_mfma.hip).
hipError_t launch_mfma_dense(const uint16_t* A, const uint16_t* B, const float* bias, int act,
                             uint16_t* C, int M, int K, int N, int cus, hipStream_t s);

// ZAYA1-style MLP router (mlp_router.hip): down-projection, depth averaging,
// RMS norm, two GELU layers, output layer + controller bias, then the usual
// softmax / top-k.  ws holds u, z [T][r], h1, h2 [T][m] bf16 and [E] fp32.
size_t mlp_router_workspace_bytes(long long T, int r, int m, int E);
hipError_t launch_route_mlp(const uint16_t* x, const uint16_t* prev, float gamma, float eps,
                            const uint16_t* wd, const float* bd, const uint16_t* w1,
                            const float* b1, const uint16_t* w2, const float* b2,
                            const uint16_t* w3, const float* b3, const float* pid,
                            float* logits, int32_t* idx, float* gate, long long T, int d, int r,
                            int m, int E, TopkParams tp, void* ws, int cus,
                            hipStream_t s);

// Gate-weighted combine.
hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* row_of,
                          const float* gate, void* y, long long T, int d, int k,
                          hipStream_t s);

// Backward GEMMs (gemm_bw.hip), fp32 results; cus = workgroups of the
// persistent grid (a multiple of 8).
// NT: nsrc (1 or 2: A1 == nullptr or not) sources times ksplit K slices,
// each an independent part p writing C + p * part_stride ([rows][N] fp32):
// part p = C_p[r][N] = A_s[r][slice] W_s[e][N][slice]^T over the rows r of
// each expert (s = p / ksplit); the sum over the parts is the product.
// bw_nt_ksplit picks ksplit so that the parts fill the chip.
int bw_nt_ksplit(long long max_rows, int E, int N, int K, int nsrc, int cus);
hipError_t launch_bw_nt(const uint16_t* A0, const uint16_t* W0, const uint16_t* A1,
                        const uint16_t* W1, float* C, long long part_stride, int ksplit,
                        const int32_t* off, int E, int N, int K, long long max_rows, int cus,
                        hipStream_t s);
// TN: C[e][M][N] = sum over the rows r of expert e of A[r][m] B[r][n]: the
// weight gradients, a ragged reduction length per expert; experts with no
// rows get zeros.
// dh_raw = A W^T (one K slice) with the GeGLU backward in the epilogue: G, U
// (bf16 [rows][N]) become dG, dU in place, gH = gate h, and
// dot[row][N / 64] the partial sums of h . dh_raw over 64-column groups.
// N % 64 == 0.
hipError_t launch_bw_nt_geglu(const uint16_t* A, const uint16_t* W, uint16_t* G, uint16_t* U,
                              uint16_t* gH, const float* row_gate, float* dot,
                              const int32_t* off, int E, int N, int K, long long max_rows,
                              int cus, hipStream_t s);
hipError_t launch_bw_tn(const uint16_t* A, const uint16_t* B, float* C, const int32_t* off,
                        int E, int M, int N, int cus, hipStream_t s);

// Backward elementwise and router kernels (backward.hip).
// The gate of each kept row (row_gate[r] = gate of the assignment that owns
// row r), and dgate_row[r] = sum of its np partials in order.
hipError_t launch_row_gate(const int32_t* offset, const int32_t* token_of_row,
                           const int32_t* row_of, const float* gate, int E, int k,
                           long long max_rows, float* row_gate, hipStream_t s);
hipError_t launch_dgate_sum(const float* dot, int np, const int32_t* offset, int E,
                            long long max_rows, float* dgate_row, hipStream_t s);
hipError_t launch_router_bwd(const float* logits, const int32_t* idx, const float* gate,
                             const int32_t* row_of, const float* dgate_row, long long T, int E,
                             int k, float tau, int renorm, float* dl, float* dgate,
                             hipStream_t s);
// dx = sum over the nparts buffers dXp + p * part_stride of the kept rows of
// each token, plus dl W_r^T.
hipError_t launch_dx(const float* dl, const uint16_t* wr, const float* dXp, int nparts,
                     long long part_stride, const int32_t* row_of, uint16_t* dx, long long T,
                     int d, int E, int k, hipStream_t s);
size_t dwr_workspace_bytes(long long T, int d, int E);
hipError_t launch_dwr(int dtype, const void* x, const float* dl, float* dwr, float* dbias,
                      long long T, int d, int E, void* ws, hipStream_t s);
// fp32 layers' backward products (backward_f32.hip): NT with an optional
// second source, NT dh_raw with the GeGLU backward in its epilogue (G, U, gH
// fp32; dot as for bf16), TN weight gradients, dx; and the recompute of g, u
// (gemm.hip).
hipError_t launch_bw_nt_f32(const float* A, const float* W, const float* A2, const float* W2,
                            float* C, const int32_t* off, int E, int N, int K, long long max_rows,
                            int cus, hipStream_t s);
hipError_t launch_bw_nt_geglu_f32(const float* A, const float* W, float* G, float* U, float* gH,
                                  const float* row_gate, float* dot, const int32_t* off, int E,
                                  int N, int K, long long max_rows, int cus, hipStream_t s);
hipError_t launch_bw_tn_f32(const float* A, const float* B, float* C, const int32_t* off, int E,
                            int M, int N, int cus, hipStream_t s);
hipError_t launch_dx_f32(const float* dl, const float* wr, const float* dXp,
                         const int32_t* row_of, float* dx, long long T, int d, int E, int k,
                         hipStream_t s);
hipError_t launch_gate_up_pre_f32(const float* x_perm, const int32_t* off, const float* w_gate,
                                  const float* w_up, float* g, float* u, int E, int d, int d_ff,
                                  long long max_rows, int grid_cap, hipStream_t s);
hipError_t launch_zero_f32(float* p, long long n, hipStream_t s);

}  // namespace moe
