// Internal launcher interface between the C ABI (tg_api.cpp) and the kernels.
// Arguments reaching these functions are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tokengate.h"

namespace tg {

// Per-request layout of a packed batch, passed to kernels by value.
struct BatchArgs {
    int32_t batch;
    int32_t cu_seq[TG_MAX_BATCH + 1];   // token offsets of each request
    int32_t cu_kept[TG_MAX_BATCH + 1];  // kept-row offsets of each request
    int32_t q_len[TG_MAX_BATCH];        // question tail length of each request
    int32_t p_len[TG_MAX_BATCH];        // template prefix length of each request (kept)
};

hipError_t launch_gate_f32(const float* hidden, int64_t T, int d, const float* w1, const float* b1,
                           const float* w2, const float* b2, int dg, float* scores, hipStream_t st);
hipError_t launch_gate_bf16(const void* hidden, int64_t T, int d, const void* w1, const void* b1,
                            const void* w2, const void* b2, int dg, float* scores, hipStream_t st);

// Selector implementation: SELECT_AUTO picks the one-workgroup path when
// every document has at most SELECT_ONE_WG_AUTO tokens, else the chunked path;
// SELECT_ONE_WG can be forced up to SELECT_ONE_WG_MAX tokens per document.
enum SelectPath { SELECT_AUTO = 0, SELECT_ONE_WG = 1, SELECT_CHUNKED = 2 };
constexpr int SELECT_ONE_WG_MAX = 65536;
constexpr int SELECT_ONE_WG_AUTO = 32768;
bool select_one_wg_fits(const BatchArgs& a, int max_doc = SELECT_ONE_WG_MAX);
inline bool select_auto_one_wg(const BatchArgs& a) { return select_one_wg_fits(a, SELECT_ONE_WG_AUTO); }
size_t select_workspace_bytes(const BatchArgs& a);
hipError_t launch_select(const float* scores, const BatchArgs& a, int32_t* kept, int32_t* cu_dev,
                         void* ws, int path, hipStream_t st);
// Device address of the library's select scratch array (TG_SELECT_SCRATCH_BYTES)
// on the device of stream st, looked up once per device.
hipError_t select_scratch(hipStream_t st, void** out);

hipError_t launch_gather(const void* hidden, int64_t T, int row_bytes, const float* scores,
                         const int32_t* kept, int64_t Kt, void* hidden_kept, float* scores_kept,
                         hipStream_t st);

struct AttnShape {
    int32_t batch;
    int32_t Hq, Hkv, d_head;
    int64_t Kt;
    int32_t cu[TG_MAX_BATCH + 1];
};

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, const float* s,
                           const float* gain, const float* temp, const AttnShape& sh, float* out,
                           float* lse, hipStream_t st);
// ws (attn_prefill_workspace_bytes, zeroed before its first use, or NULL)
// lets a single request whose grid cannot fill the chip cut its query tiles
// into pieces of at most 8 key tiles, one workgroup each.
size_t attn_prefill_workspace_bytes(const AttnShape& sh);
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, const float* s,
                            const float* gain, const float* temp, const AttnShape& sh, void* out,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t st);

size_t attn_bwd_workspace_bytes(const AttnShape& sh);
hipError_t launch_attn_bwd(const AttnShape& sh, const void* q, const void* k, const void* v,
                           const float* s, const float* gain, const float* temp, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* ds, float* dgain, float* dtemp, void* ws, hipStream_t st);

size_t gate_bwd_workspace_bytes(tg_dtype dt, int64_t Kt, int d, int dg);
hipError_t launch_gate_bwd(tg_dtype dt, const void* x, int64_t Kt, int d, const void* w1,
                           const void* b1, const void* w2, int dg, const float* ds, void* dx,
                           void* dw1, float* db1, float* dw2, float* db2, void* ws,
                           hipStream_t st);

struct DecodeShape {
    int32_t batch;
    int32_t Hq, Hkv, d_head;
    int32_t max_len;
    int64_t rows;  // rows in the K/V/score pool
};

size_t decode_workspace_bytes(int32_t batch, int32_t Hq, int32_t d_head, int32_t max_len);
hipError_t launch_decode(tg_dtype dt, const DecodeShape& sh, const void* q, const void* k,
                         const void* v, const float* s, const int64_t* row_off,
                         const int32_t* cache_len, const float* gain, const float* temp, void* out,
                         float* lse, void* ws, hipStream_t st);

hipError_t launch_rmsnorm(tg_dtype dt, const void* x, const void* w, float eps, int64_t M, int d,
                          void* y, hipStream_t st);
hipError_t launch_qk_norm_rope(tg_dtype dt, void* q, void* k, const void* qw, const void* kw,
                               const int32_t* pos, int64_t M, int Hq, int Hkv, int dh, float theta,
                               float eps, hipStream_t st);
hipError_t launch_silu_mul(tg_dtype dt, const void* gu, int64_t M, int F, void* out,
                           hipStream_t st);
hipError_t launch_kept_positions(const int32_t* kept, int64_t Kt, const BatchArgs& a, int32_t* pos,
                                 hipStream_t st);

hipError_t launch_linear_f32(const float* x, const float* w, float* y, int64_t M, int N, int K,
                             int accumulate, hipStream_t st);
// tile: 0 chooses by output size; 1, 2, 3 force the 128x128, 256x128, 256x256 tile.
// Products of one x with up to LINEAR_MAX_SEG weights in one launch; every
// n[i] a multiple of 256 when nseg > 1.
constexpr int LINEAR_MAX_SEG = 3;
hipError_t launch_linear_bf16_multi(const void* x, int nseg, const void* const* w, void* const* y,
                                    const int* n, int64_t M, int K, int accumulate, int tile,
                                    hipStream_t st);
// out[M][F] = silu(x wgu[0:F]^T) * (x wgu[F:2F]^T); F a multiple of 128.
hipError_t launch_linear_bf16_swiglu(const void* x, const void* wgu, void* out, int64_t M, int F,
                                     int K, int tile, hipStream_t st);
hipError_t launch_linear_bf16(const void* x, const void* w, void* y, int64_t M, int N, int K,
                              int accumulate, int tile, hipStream_t st);
// part[z][M][N] = x[:, zK/S : (z+1)K/S] . w[:, same]^T in fp32, z < S (K/S a multiple of 64).
hipError_t launch_linear_bf16_splitk(const void* x, const void* w, float* part, int64_t M, int N,
                                     int K, int slices, hipStream_t st);

}  // namespace tg
