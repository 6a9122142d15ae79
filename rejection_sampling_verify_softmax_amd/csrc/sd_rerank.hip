// sd_rerank.hip -- EAGLE-2-style choice of the verification tree.
//
// Page "大模型投机解码：Medusa、MTP、EAGLE、DFlash、DDTree 与 DSpark"
// (chzhyang.github.io), §4 EAGLE-2: candidates are expanded along paths of high
// cumulative confidence, then re-ranked, and the final verification tree is
// chosen from them (its depth and width follow the context).
//
// Input per sequence: an expanded candidate tree in topological order
// (candidate 0 the root, every other candidate's parent an earlier one) with
// each candidate's token and conditional draft probability. Its cumulative
// confidence is the fp32 product of the conditional probabilities along its
// path, root first. The tree keeps the root plus the N-1 best candidates by
// (confidence desc, depth asc, candidate index asc); a child never beats its
// parent under that order, so the kept set is closed under taking parents.
// Nodes are numbered in that order, with the outputs of the DDTree build.
//
// One workgroup per sequence: level-synchronous confidences in LDS; each wave
// sorts the 64-bit keys of its quarter of the candidates, and the four lists'
// heads merge by rank into the kept nodes; then one thread per kept node.
#include "sd_device.hpp"
#include "sd_internal.hpp"

namespace sd {

namespace {

constexpr int kMaxCand = 1024;
constexpr int kCandPerThread = kMaxCand / kBlock;

__device__ __forceinline__ uint32_t conf_bits(float x) {
    // x in [0, 1]: its bits order it (no negatives, no NaN)
    return __float_as_uint(x);
}

__global__ __launch_bounds__(kBlock) void k_rerank_tree(
    const int32_t* __restrict__ cand_parent, const int32_t* __restrict__ cand_token,
    const float* __restrict__ cand_prob, const int32_t* __restrict__ n_cand, int M, int N,
    int32_t* __restrict__ node_token, int32_t* __restrict__ node_parent,
    int32_t* __restrict__ node_depth, float* __restrict__ node_score,
    unsigned long long* __restrict__ node_anc, int32_t* __restrict__ node_cand,
    int32_t* __restrict__ n_nodes) {
    __shared__ float score[kMaxCand];
    __shared__ int par[kMaxCand];
    __shared__ int depth[kMaxCand];
    __shared__ unsigned char ready[kMaxCand];
    __shared__ unsigned long long wkeys[kWavesPerBlock][kWave * kCandPerThread];
    __shared__ unsigned long long top[64];
    __shared__ int node_of[kMaxCand];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    int nc = n_cand[b];
    nc = nc < 0 ? 0 : (nc > M ? M : nc);
    const int64_t o = (int64_t)b * M;
    // 1. candidates: a bad parent or probability leaves a candidate (and its
    //    subtree) out
    float prob[kCandPerThread];
#pragma unroll
    for (int j = 0; j < kCandPerThread; ++j) {
        const int i = j * kBlock + tid;
        int p = -1;
        float q = 0.f;
        if (i < nc && i > 0) {
            p = cand_parent[o + i];
            q = cand_prob[o + i];
        }
        const bool ok = i > 0 && i < nc && p >= 0 && p < i && q >= 0.f && q <= 1.f;
        par[i] = ok ? p : -1;
        prob[j] = q;
        ready[i] = (i == 0 && nc > 0) ? 1 : 0;
        score[i] = (i == 0) ? 1.0f : 0.f;
        depth[i] = 0;
        node_of[i] = (i == 0) ? 0 : -1;
    }
    __syncthreads();
    // 2. confidences level by level: a candidate is done once its parent is
    //    (read, then write, so one level never sees its own updates)
    bool more = true;
    while (more) {
        bool mine[kCandPerThread];
        float ns[kCandPerThread];
        int nd[kCandPerThread];
        bool any = false;
#pragma unroll
        for (int j = 0; j < kCandPerThread; ++j) {
            const int i = j * kBlock + tid;
            const int p = par[i];
            mine[j] = !ready[i] && p >= 0 && ready[p];
            ns[j] = mine[j] ? score[p] * prob[j] : 0.f;
            nd[j] = mine[j] ? depth[p] + 1 : 0;
            any = any || mine[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kCandPerThread; ++j) {
            const int i = j * kBlock + tid;
            if (mine[j]) {
                score[i] = ns[j];
                depth[i] = nd[j];
                ready[i] = 1;
            }
        }
        more = __syncthreads_or(any) != 0;
    }
    // 3. keys: (confidence desc, depth asc, index asc); 0 = not a candidate.
    //    Each wave sorts its own candidates' keys; a key among the first N-1
    //    of its wave's list takes its rank from its place there plus, by
    //    binary search, the keys above it in the other waves' first N-1.
    const int w = tid / kWave, lane = tid & (kWave - 1);
    unsigned long long* wk = wkeys[w];
#pragma unroll
    for (int j = 0; j < kCandPerThread; ++j) {
        const int i = j * kBlock + tid;
        wk[lane * kCandPerThread + j] =
            (i > 0 && ready[i]) ? ((unsigned long long)conf_bits(score[i]) << 32) |
                                      ((unsigned long long)(0xffff - depth[i]) << 16) |
                                      (unsigned long long)(0xffff - i)
                                : 0ull;
    }
    wave_sort_desc(wk, kWave * kCandPerThread);
    const int kept_max = N - 1;
    if (tid < 64) top[tid] = 0ull;
    __syncthreads();
    for (int p = lane; p < kept_max; p += kWave) {
        const unsigned long long key = wk[p];
        if (key != 0ull) {
            int rank = p;
            for (int o = 0; o < kWavesPerBlock; ++o)
                if (o != w) rank += count_above(wkeys[o], kept_max, key);
            if (rank < kept_max) top[rank] = key;
        }
    }
    __syncthreads();
    // 4. the first N-1 keys are the kept nodes, numbered in order
    if (tid < kept_max && top[tid] != 0ull) node_of[0xffff - (int)(top[tid] & 0xffffull)] = tid + 1;
    __syncthreads();
    const int64_t on = (int64_t)b * N;
    if (tid < N) {
        int tok = -1, pn = -1, dep = 0, cand = 0;
        float sc = 1.0f;
        unsigned long long anc = 1ull;
        if (tid > 0) {
            const unsigned long long key = top[tid - 1];
            if (key != 0ull) {
                cand = 0xffff - (int)(key & 0xffffull);
                tok = cand_token[o + cand];
                pn = node_of[par[cand]];
                dep = depth[cand];
                sc = score[cand];
                anc = 1ull << tid;
                for (int c = par[cand]; c > 0; c = par[c]) anc |= 1ull << node_of[c];
                anc |= 1ull;                                   // the root
            } else {
                cand = -1;
                sc = 0.f;
                anc = 0ull;
            }
        }
        node_token[on + tid] = tok;
        node_parent[on + tid] = pn;
        node_depth[on + tid] = dep;
        node_score[on + tid] = sc;
        node_anc[on + tid] = anc;
        if (node_cand) node_cand[on + tid] = cand;
    }
    if (tid == 0) {
        int k = 0;
        while (k < kept_max && top[k] != 0ull) ++k;
        n_nodes[b] = 1 + k;
    }
}

}  // namespace

hipError_t launch_rerank_tree(const int32_t* cand_parent, const int32_t* cand_token,
                              const float* cand_prob, const int32_t* n_cand, int B, int M, int N,
                              int32_t* tok, int32_t* par, int32_t* dep, float* score, uint64_t* anc,
                              int32_t* node_cand, int32_t* n_nodes, hipStream_t stream) {
    PassTimer::launch(k_rerank_tree, dim3(B), dim3(kBlock), stream, cand_parent, cand_token,
                      cand_prob, n_cand, M, N, tok, par, dep, score,
                      reinterpret_cast<unsigned long long*>(anc), node_cand, n_nodes);
    return hipGetLastError();
}

}  // namespace sd
