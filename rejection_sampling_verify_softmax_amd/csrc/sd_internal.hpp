// sd_internal.hpp -- host-side launch interface between the ABI layer and the
// kernel files of libsd. Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sd {

// Elements of one row handled by one workgroup of the streaming kernels.
// Multiples of kBlock * 16-byte vectors so that chunk boundaries are vector
// aligned.
constexpr int kMaxTopk = 256;
constexpr int kMaxTreeK = 16;
#ifndef SD_CHUNK_BF16
#define SD_CHUNK_BF16 32768
#endif
#ifndef SD_CHUNK_F32
#define SD_CHUNK_F32 16384
#endif
constexpr int kChunkBf16 = SD_CHUNK_BF16;
constexpr int kChunkF32 = SD_CHUNK_F32;
static_assert(kChunkBf16 % (256 * 8) == 0, "bf16 chunk: whole workgroup rounds of 16-byte vectors");
static_assert(kChunkF32 % (256 * 4) == 0, "fp32 chunk: whole workgroup rounds of 16-byte vectors");

inline int chunk_elems(int dtype) { return dtype == 1 ? kChunkBf16 : kChunkF32; }
inline int n_chunks_for(int V, int dtype) {
    const int c = chunk_elems(dtype);
    return (V + c - 1) / c;
}

// Sub-allocation of the caller's workspace: 256-byte aligned regions.
struct Carve {
    size_t off = 0;
    size_t take(size_t bytes) {
        size_t o = off;
        off += (bytes + 255) & ~size_t(255);
        return o;
    }
};

// Optional events for the streaming kernel of the next call on this thread
// (set by sd_time_next_stream_pass). launch() binds them to that kernel's own
// dispatch (hipExtLaunchKernel: the events take the kernel's start and end
// times, with no marker packets between it and its neighbours on the stream)
// and clears them; mark_before()/mark_after() record them directly, for a call
// that launches no streaming kernel.
struct PassTimer {
    static thread_local hipEvent_t start;
    static thread_local hipEvent_t stop;
    template <typename F, typename... Args>
    static void launch(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
        hipEvent_t a = start, b = stop;
        start = stop = nullptr;
        hipExtLaunchKernelGGL(kernel, grid, block, 0, s, a, b, 0, args...);
    }
    static void mark_before(hipStream_t s) {
        if (start) (void)hipEventRecord(start, s);
        start = nullptr;
    }
    static void mark_after(hipStream_t s) {
        if (stop) (void)hipEventRecord(stop, s);
        stop = nullptr;
    }
};

struct ChainArgs {
    const void* target;
    const void* draft;
    int dtype;                 // 0 f32, 1 bf16
    const int32_t* tokens;
    const float* uniforms;
    const int32_t* cu;
    int B, K_max, V;
    float temperature;
    int top_k;
    int32_t* accepted_len;
    int32_t* next_token;
    float* probs_out;
    float* resid_mass_out;
    int32_t* seq_status;
    const int32_t* cap;        // per-sequence cap on the committed length, or nullptr
    int32_t* accepted_full;    // first rejection over the whole window (with cap), or nullptr
    void* ws;
    hipStream_t stream;
};

// Workspace bytes of each path (all sizes already validated).
size_t chain_full_ws_bytes(int B, int K_max, int V, int dtype);
size_t chain_topk_ws_bytes(int B, int K_max, int V, int top_k);
size_t greedy_ws_bytes(int B, int K_max, int V, int dtype);
size_t tree_build_ws_bytes(int B, int K, int V, int N);

hipError_t launch_chain_full(const ChainArgs& a);
hipError_t launch_chain_topk(const ChainArgs& a);
hipError_t launch_greedy(const void* target, int dtype, const int32_t* tokens, const int32_t* cu,
                         int B, int K_max, int V, int32_t* accepted_len, int32_t* next_token,
                         int32_t* seq_status, const int32_t* cap, int32_t* accepted_full, void* ws,
                         hipStream_t stream);
hipError_t launch_tree_build(const float* marg, int B, int K, int V, int N, int32_t* tok,
                             int32_t* par, int32_t* dep, float* score, uint64_t* anc,
                             int32_t* n_nodes, void* ws, hipStream_t stream);
hipError_t launch_tree_walk_rows(const void* target, int dtype, const int32_t* tok,
                                 const int32_t* par, const int32_t* n_nodes, const float* uniforms,
                                 int B, int N, int V, float temperature, int32_t* path,
                                 int32_t* accepted_len, int32_t* next_token, int32_t* seq_status,
                                 hipStream_t stream);
hipError_t launch_tree_walk_topk(const void* target, int dtype, const int32_t* tok, const int32_t* par,
                                 const int32_t* n_nodes, const float* uniforms, int B, int N, int V,
                                 float temperature, int top_k, int32_t* path, int32_t* accepted_len,
                                 int32_t* next_token, int32_t* seq_status, hipStream_t stream);
hipError_t launch_compact_kv(void* kv, int64_t row_bytes, int64_t n_rows, const int64_t* base,
                             const int32_t* path, const int32_t* accepted_len, int B, int N,
                             hipStream_t stream);
hipError_t launch_rerank_tree(const int32_t* cand_parent, const int32_t* cand_token,
                              const float* cand_prob, const int32_t* n_cand, int B, int M, int N,
                              int32_t* tok, int32_t* par, int32_t* dep, float* score, uint64_t* anc,
                              int32_t* node_cand, int32_t* n_nodes, hipStream_t stream);
hipError_t launch_expand_tree(int32_t* cand_parent, int32_t* cand_token, float* cand_prob,
                              float* cand_conf, int32_t* n_cand, const int32_t* expand_in,
                              int32_t* expand_out, const int32_t* child_token, const float* child_prob,
                              int B, int M, int W, int C, hipStream_t stream);
hipError_t launch_stream_read(const void* data, int64_t bytes, uint32_t* sink, int n_blocks,
                              hipStream_t stream);
hipError_t launch_stream_read_rows(const void* data, int64_t row_bytes, int n_rows, int64_t chunk_bytes,
                                   uint32_t* sink, hipStream_t stream);
hipError_t launch_select_len(const float* conf, int B, int K_max, float cost, const float* table,
                             int32_t* k_sel, float* adv, int32_t* cu_sel, hipStream_t stream);

}  // namespace sd
