// plan.hip -- skew-balancing plan over logical rank partitions + block table (moe_plan).
//
// MoonEP routing flow ("Same data, summed per rank" and "The greedy balance, step by step"):
// a rank's surplus is its experts' entries minus its capacity S*K; each move refills the
// currently hungriest rank in one shot from the currently biggest donor, the donor may
// overshoot below capacity and be refilled later, and a move is realised by slicing the
// donor's biggest experts.  MegaFlux §3.1 / App. A.2: the plan keeps every selection; each
// expert's rows are cut into blocks of at most beta rows in the expert's stable order.
//
// One workgroup.  The greedy is sequential by nature (at most P-1 rank moves, each a few
// slices) and runs in wave 0: lane r holds rank r's surplus in a register, the experts'
// remaining counts sit in LDS.  Arg-min / arg-max run only over the lanes that compete (the
// P ranks, or the donor's G = E_loc / P experts, one per lane) under total orders (value,
// then lowest id), so ties resolve exactly as stated in moe.h; groups of up to 16 lanes
// reduce with DPP lane swaps inside a row, larger ones add cross-row shuffles.  The block
// table is then emitted by all threads from a scan of per-(rank, expert) block counts.
#include "moe_launch.h"
#include "moe_wave.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxSlices = 4096;  // E_loc * P

__global__ void __launch_bounds__(kThreads)
plan_kernel(const int32_t* __restrict__ counts, int begin, int stride, int E_loc, int P,
            int beta, int32_t* __restrict__ q_out, int32_t* __restrict__ moves,
            int32_t* __restrict__ n_moves, int max_moves, int32_t* __restrict__ blocks,
            int32_t* __restrict__ n_blocks, int max_blocks, int32_t* __restrict__ err_word) {
    __shared__ int n_s[256];
    __shared__ int rem_s[256];
    __shared__ int off_s[257];
    __shared__ int q_s[kMaxSlices];      // [l * P + r]
    __shared__ int start_s[kMaxSlices];  // first row of slice (l, r), then its first block
    __shared__ int part[kThreads / MOE_WAVE];
    __shared__ int err_s;

    const int tid = threadIdx.x;
    const int lane = moe_lane_id();
    const int G = E_loc / P;

    for (int l = tid; l < E_loc; l += kThreads) {
        const int n = counts[begin + l * stride];
        n_s[l] = n;
        rem_s[l] = n;
    }
    for (int i = tid; i < E_loc * P; i += kThreads) q_s[i] = 0;
    if (tid == 0) err_s = 0;
    __syncthreads();

    if (tid < MOE_WAVE) {
        // padded segment starts (same layout as moe_permute) and N, by a wave scan
        int padded[4], raw = 0, pad_sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int l = lane * 4 + j;
            int n = l < E_loc ? n_s[l] : 0;
            padded[j] = (n + beta - 1) / beta * beta;
            pad_sum += padded[j];
            raw += n;
        }
        int incl = pad_sum;
#pragma unroll
        for (int d = 1; d < MOE_WAVE; d <<= 1) {
            int o = __shfl_up(incl, d, MOE_WAVE);
            if (lane >= d) incl += o;
        }
        int run = incl - pad_sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int l = lane * 4 + j;
            if (l < E_loc) off_s[l] = run;
            run += padded[j];
        }
        if (lane == MOE_WAVE - 1) off_s[E_loc] = incl;
        const int N = moe_wave_sum_i32(raw);

        // surplus of rank `lane`
        int d = 0;
        if (lane < P) {
            int load = 0;
            for (int l = lane * G; l < (lane + 1) * G; ++l) load += n_s[l];
            d = load - (N / P + (lane < N % P ? 1 : 0));
        }
        const int rank_levels = ceil_log2(P);
        const int gsize = G < MOE_WAVE ? G : MOE_WAVE;
        const int expert_levels = ceil_log2(gsize);
        int nm = 0, err = 0;
        for (int iter = 0; iter <= P; ++iter) {
            int mn = lane < P ? d : 0x7FFFFFFF, mn_i = lane;
            int mx = lane < P ? d : (int)0x80000000, mx_i = lane;
            group_best<false>(mn, mn_i, rank_levels);
            group_best<true>(mx, mx_i, rank_levels);
            mn = __builtin_amdgcn_readfirstlane(mn);
            mn_i = __builtin_amdgcn_readfirstlane(mn_i);
            mx_i = __builtin_amdgcn_readfirstlane(mx_i);
            if (mn >= 0) break;
            if (iter == P) {  // cannot happen: each move settles one rank for good
                err |= 4;
                break;
            }
            const int recv = mn_i, donor = mx_i;
            int need = -mn;
            if (lane == donor) d -= need;
            if (lane == recv) d = 0;
            for (int s = 0; need > 0; ++s) {
                // donor's own expert with the most remaining entries (lowest id on ties):
                // lane i looks at experts donor*G + i, + 64, ...
                int bv = 0, bl = 0x7FFFFFFF;
                for (int l = donor * G + lane; l < (donor + 1) * G; l += MOE_WAVE) {
                    const int r = rem_s[l];
                    if (r > 0 && (r > bv || (r == bv && l < bl))) {
                        bv = r;
                        bl = l;
                    }
                }
                group_best<true>(bv, bl, expert_levels);
                bv = __builtin_amdgcn_readfirstlane(bv);
                bl = __builtin_amdgcn_readfirstlane(bl);
                if (bv <= 0 || s > G) {  // cannot happen: a donor always covers its move
                    err |= 4;
                    break;
                }
                const int take = bv < need ? bv : need;
                if (lane == 0) {
                    rem_s[bl] = bv - take;
                    q_s[bl * P + recv] += take;
                    if (nm < max_moves) {
                        moves[4 * nm + 0] = donor;
                        moves[4 * nm + 1] = recv;
                        moves[4 * nm + 2] = bl;
                        moves[4 * nm + 3] = take;
                    }
                }
                ++nm;
                need -= take;
            }
            if (err) break;
        }
        if (nm > max_moves) err |= 2;
        // leftovers stay with the owner
        for (int l = lane; l < E_loc; l += MOE_WAVE) q_s[l * P + l / G] += rem_s[l];
        if (lane == 0) {
            *n_moves = nm < max_moves ? nm : max_moves;
            err_s = err;
        }
    }
    __syncthreads();

    for (int i = tid; i < E_loc * P; i += kThreads) q_out[i] = q_s[i];
    // first row of slice (l, r): segment start + rows of expert l taken by lower ranks
    for (int l = tid; l < E_loc; l += kThreads) {
        int acc = off_s[l];
        for (int r = 0; r < P; ++r) {
            start_s[l * P + r] = acc;
            acc += q_s[l * P + r];
        }
    }
    __syncthreads();

    // blocks per slice, slices in table order s = r * E_loc + l; thread owns a run of slices
    const int S = E_loc * P;
    const int per = (S + kThreads - 1) / kThreads;
    const int s_begin = min(S, tid * per);
    const int s_end = min(S, s_begin + per);
    int cnt = 0;
    for (int s = s_begin; s < s_end; ++s) {
        int r = s / E_loc, l = s - r * E_loc;
        cnt += (q_s[l * P + r] + beta - 1) / beta;
    }
    // exclusive scan of the per-thread block counts: within each wave by shuffles, across
    // the four waves through LDS
    int incl = cnt;
#pragma unroll
    for (int dd = 1; dd < MOE_WAVE; dd <<= 1) {
        const int o = __shfl_up(incl, dd, MOE_WAVE);
        if (lane >= dd) incl += o;
    }
    const int wave = tid / MOE_WAVE;
    if (lane == MOE_WAVE - 1) part[wave] = incl;
    __syncthreads();
    int b = incl - cnt, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / MOE_WAVE; ++w) {
        b += w < wave ? part[w] : 0;
        total += part[w];
    }
    for (int s = s_begin; s < s_end; ++s) {
        int r = s / E_loc, l = s - r * E_loc;
        int take = q_s[l * P + r];
        int first = start_s[l * P + r];
        for (int j = 0; j * beta < take; ++j, ++b) {
            if (b < max_blocks) {
                int rows = take - j * beta < beta ? take - j * beta : beta;
                blocks[4 * b + 0] = r;
                blocks[4 * b + 1] = l;
                blocks[4 * b + 2] = first + j * beta;
                blocks[4 * b + 3] = rows;
            }
        }
    }
    if (tid == 0) {
        int err = err_s;
        if (total > max_blocks) err |= 1;
        *n_blocks = total < max_blocks ? total : max_blocks;
        if (err_word) *err_word = err;
    }
}

}  // namespace

hipError_t moe_launch_plan(const int32_t* counts, int begin, int stride, int E_loc, int P,
                           int beta, int32_t* q, int32_t* moves, int32_t* n_moves,
                           int max_moves, int32_t* blocks, int32_t* n_blocks, int max_blocks,
                           int32_t* err_word, hipStream_t stream) {
    plan_kernel<<<1, kThreads, 0, stream>>>(counts, begin, stride, E_loc, P, beta, q, moves,
                                            n_moves, max_moves, blocks, n_blocks, max_blocks,
                                            err_word);
    return hipGetLastError();
}
