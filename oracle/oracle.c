/*
 * oracle.c -- plain, slow CPU reference of the routed-expert path of one MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link, load or
 * call this file.  It exists so that tests, the smoke check and the CPU-baseline leg of
 * the benchmark can check the GPU library against an independent implementation.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * Every step is the plain definition of what the path computes, written as loops in the
 * order the source pages state them.  Floating point is accumulated in double; the two
 * rounding points that the bf16 path has (the SwiGLU activation and the expert output,
 * plus the final combined output) round the double result to bf16, nearest-even.
 *
 * Sources (the pages' titles and the parts used):
 *   [MF]   "MegaFlux: Skew-Resilient MoE Megakernels via Pipelined Expert Replication":
 *          §1 (router picks k experts, outputs combined by routing weights),
 *          §2.1 (FC1 -> FC2 SwiGLU experts; the final top-k sum is its own launch),
 *          §3.1 (blocks of at most beta rows; stable order inside each expert),
 *          §4.1 (beta = 128, SwiGLU, FP32 accumulation with BF16 outputs; k distinct experts),
 *          App. A.2 (assignments ordered by source and (token, top-k position); ids, positions
 *          and weights kept for the combine), App. B.2 (routed work is conserved).
 *   [MEP]  "MoonEP routing flow -- live": the per-rank surplus over capacity S*K, and the
 *          greedy balance (hungriest receiver refilled in one shot from the biggest donor,
 *          donor may overshoot, moves realised by slicing the donor's biggest experts).
 *   [RN]   Daily Papers listing, the abstract on top-k renormalisation in fine-grained MoEs
 *          (probabilities of the selected experts are renormalised).
 *
 * Parity status per function is stated in each header comment ("pinned by" lists the
 * CPU tests that tie the function to something other than itself).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_DATA 2

/* ---------------------------------------------------------------- bf16 helpers --- */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, straight from the definition:
 * bf16 keeps 8 significant bits.  Writing v = m * 2^e with 0.5 <= |m| < 1, the nearest
 * value is nearbyint(m * 2^8) * 2^(e-8) (nearbyint rounds ties to even in the default
 * rounding mode).  Valid for |v| in the normal binary32 range, which is all the path
 * produces; zero keeps its sign.  Pinned by: test_oracle_pins.py::test_bf16_rounding. */
uint16_t oracle_double_to_bf16(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
    int e;
    double m = frexp(v, &e);
    double r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* Element i of an array of dtype dt (0 = float32, 1 = bf16), widened to double. */
static double load_elem(const void* p, int64_t i, int dt) {
    if (dt == 1) return bf16_bits_to_double(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

/* Store a double into element i of an array of dtype dt, rounding to nearest-even.
 * (double -> float conversion in C rounds to nearest-even.) */
static void store_elem(void* p, int64_t i, int dt, double v) {
    if (dt == 1)
        ((uint16_t*)p)[i] = oracle_double_to_bf16(v);
    else
        ((float*)p)[i] = (float)v;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the oracle's parallel loops from now on (n >= 1); returns the new count. */
int oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return oracle_num_threads();
}

/* ------------------------------------------------------------------------ route --- */

/* Router top-k and routing weights.  [MF §1]: each token is sent to k experts and their
 * outputs are mixed with routing weights; [MF §4.1]: the k experts of a token are distinct;
 * [RN]: the probabilities of the picked experts are renormalised over the picks.
 *
 * For token t the experts are ranked by the key (larger logit first, then smaller expert
 * id); ids[t][0..K) are the first K in that order (slot 0 = the largest).  Weights are the
 * softmax of the logits: renormalize != 0 -> over the K picks, else over all E experts.
 * The maximum logit is subtracted before exp (it cancels in the ratio).  counts[e] is the
 * number of (t, k) with ids[t][k] == e.
 * Pinned by: full stable sort per row (ids), torch.softmax in float64 (weights), sums. */
int oracle_route(const float* logits, int T, int E, int K, int renormalize,
                 int32_t* ids, float* w, int32_t* counts) {
    if (T < 1 || E < 1 || K < 1 || K > E) return ORACLE_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float* row = logits + (int64_t)t * E;
        unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
        if (!taken) { bad = 1; continue; }
        /* K selection passes; a strict '>' keeps the lower id on equal logits */
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || row[e] > row[best]) best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * K + k] = best;
        }
        free(taken);
        double m = (double)row[ids[(int64_t)t * K]];
        double denom = 0.0;
        if (renormalize) {
            for (int k = 0; k < K; ++k) denom += exp((double)row[ids[(int64_t)t * K + k]] - m);
        } else {
            for (int e = 0; e < E; ++e) denom += exp((double)row[e] - m);
        }
        for (int k = 0; k < K; ++k)
            w[(int64_t)t * K + k] = (float)(exp((double)row[ids[(int64_t)t * K + k]] - m) / denom);
    }
    if (bad) return ORACLE_ERR_DATA;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t i = 0; i < (int64_t)T * K; ++i) counts[ids[i]] += 1;
    return ORACLE_OK;
}

/* Top-k with a reference set.  [RN]: the top k_1 experts are activated while their weights
 * are normalised by the probability mass of the top k_2 experts; k_2 = k_1 is the usual
 * renormalisation over the picks and dropping renormalisation is the plain softmax over all
 * experts.  Here K = k_1 and k_ref = k_2, K <= k_ref <= E.
 *
 * ids and counts exactly as oracle_route.  With m the largest logit of the token,
 * w[t][k] = exp(l[ids[t][k]] - m) / sum over the first k_ref experts of the token's ranking of
 * exp(l - m).  For k_ref = E that set is every expert, summed in expert order.
 * Pinned by: an argsort-based float64 computation of the same ratio (every k_ref); equality
 * with oracle_route at k_ref = K and k_ref = E. */
int oracle_route_ref(const float* logits, int T, int E, int K, int k_ref, int32_t* ids,
                     float* w, int32_t* counts) {
    if (T < 1 || E < 1 || K < 1 || K > E || k_ref < K || k_ref > E) return ORACLE_ERR_ARG;
    const int picks = k_ref < E ? k_ref : K;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float* row = logits + (int64_t)t * E;
        unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
        int* order = (int*)malloc(sizeof(int) * (size_t)picks);
        if (!taken || !order) {
            bad = 1;
            free(taken);
            free(order);
            continue;
        }
        /* selection passes under (larger logit, smaller id), as in oracle_route */
        for (int k = 0; k < picks; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || row[e] > row[best]) best = e;
            }
            taken[best] = 1;
            order[k] = best;
        }
        for (int k = 0; k < K; ++k) ids[(int64_t)t * K + k] = order[k];
        double m = (double)row[order[0]];
        double denom = 0.0;
        if (k_ref < E) {
            for (int k = 0; k < k_ref; ++k) denom += exp((double)row[order[k]] - m);
        } else {
            for (int e = 0; e < E; ++e) denom += exp((double)row[e] - m);
        }
        for (int k = 0; k < K; ++k)
            w[(int64_t)t * K + k] = (float)(exp((double)row[order[k]] - m) / denom);
        free(taken);
        free(order);
    }
    if (bad) return ORACLE_ERR_DATA;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t i = 0; i < (int64_t)T * K; ++i) counts[ids[i]] += 1;
    return ORACLE_OK;
}

/* Router scores.  [TM] (the TritonMoE abstract): the forward pass starts with router scoring;
 * a linear router scores token t against expert e with the dot product of the token's
 * activation row and the expert's router row:
 *   logits[t][e] = sum over h of x[t][h] * w_r[e][h],
 * x [T, H] and w_r [E, H] of dtype dt (0 = float32, 1 = bf16), accumulated in double in
 * ascending h and rounded once to float32.
 * Pinned by: one-hot router rows reproduce columns of x exactly; scaling x by 2 scales the
 * logits by 2 exactly; a float64 library matrix product rounded to float32. */
int oracle_router_logits(const void* x, int dt, const void* w_r, int T, int H, int E,
                         float* logits) {
    if (T < 1 || H < 1 || E < 1 || (dt != 0 && dt != 1)) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += load_elem(x, (int64_t)t * H + h, dt) * load_elem(w_r, (int64_t)e * H + h, dt);
            logits[(int64_t)t * E + e] = (float)acc;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- permute --- */

/* Local index of global expert e in the set { begin + j*stride : 0 <= j < E_loc }, or -1. */
static int local_index(int e, int begin, int stride, int E_loc) {
    int d = e - begin;
    if (d < 0 || d % stride != 0) return -1;
    int l = d / stride;
    return l < E_loc ? l : -1;
}

/* Tile-aligned expert offsets: off[0] = 0, off[l+1] = off[l] + ceil(n_l / beta) * beta,
 * so every expert's segment starts on a multiple of beta.  [MF §3.1]: an expert's rows are
 * cut into blocks of at most beta rows.  Returns the padded total. */
static int64_t padded_offsets(const int32_t* counts, int begin, int stride, int E_loc, int beta,
                              int32_t* off) {
    off[0] = 0;
    for (int l = 0; l < E_loc; ++l) {
        int64_t n = counts[begin + l * stride];
        int64_t padded = (n + beta - 1) / beta * beta;
        off[l + 1] = (int32_t)(off[l] + padded);
    }
    return off[E_loc];
}

/* Dispatch permutation.  [MF §3.1, App. A.2]: inside each expert the routed assignments
 * keep a stable, deterministic order by source and (token, top-k position); with tokens
 * laid out source-major that is the flat index i = t*K + k ascending.  Entry i routed to
 * local expert l gets the next free row of l's segment; entry_pos[i] is that row (-1 when
 * the expert is not local), row_token[row] = t (-1 on padding rows), and row `row` of xp is
 * a copy of row t of x (row_bytes bytes each; x/xp may be NULL to skip the copy).
 * Returns ORACLE_ERR_DATA if counts disagree with ids.
 * Pinned by: Python sorted() over (expert, i); bijection and multiset checks. */
int oracle_permute(const int32_t* ids, const int32_t* counts, int T, int K, int E,
                   int begin, int stride, int E_loc, int beta,
                   const void* x, int64_t row_bytes,
                   int32_t* offsets, int32_t* entry_pos, int32_t* row_token, void* xp,
                   int64_t max_rows) {
    if (T < 1 || K < 1 || E < 1 || E_loc < 1 || stride < 1 || beta < 1) return ORACLE_ERR_ARG;
    if (begin < 0 || begin + (int64_t)(E_loc - 1) * stride >= E) return ORACLE_ERR_ARG;
    int64_t rows_pad = padded_offsets(counts, begin, stride, E_loc, beta, offsets);
    if (rows_pad > max_rows) return ORACLE_ERR_ARG;
    for (int64_t p = 0; p < rows_pad; ++p) row_token[p] = -1;
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E_loc);
    if (!cursor) return ORACLE_ERR_DATA;
    for (int l = 0; l < E_loc; ++l) cursor[l] = offsets[l];
    for (int64_t i = 0; i < (int64_t)T * K; ++i) {
        int l = local_index(ids[i], begin, stride, E_loc);
        if (l < 0) {
            entry_pos[i] = -1;
            continue;
        }
        int32_t p = cursor[l]++;
        int t = (int)(i / K);
        entry_pos[i] = p;
        row_token[p] = t;
        if (x && xp)
            memcpy((char*)xp + (int64_t)p * row_bytes, (const char*)x + (int64_t)t * row_bytes,
                   (size_t)row_bytes);
    }
    int rc = ORACLE_OK;
    for (int l = 0; l < E_loc; ++l)
        if (cursor[l] != offsets[l] + counts[begin + l * stride]) rc = ORACLE_ERR_DATA;
    free(cursor);
    return rc;
}

/* ------------------------------------------------------------------------- plan --- */

/* Skew-balancing plan over P logical partitions ("ranks"), which are data, not devices.
 *
 * [MEP]: each rank owns a contiguous group of G = E_loc / P experts; its surplus is the sum
 * of its experts' entries minus its capacity S*K, the number of entries it computes after
 * balancing.  Capacity here: C_r = floor(N/P) + (r < N mod P), which is S*K whenever P | N.
 * The greedy repeats, while some rank is below capacity:
 *   receiver = the rank with the lowest surplus (the hungriest), lowest id on ties;
 *   donor    = the rank with the highest surplus (the biggest donor), lowest id on ties;
 *   the receiver is refilled in one move by need = -surplus(receiver) entries: its surplus
 *   becomes 0, the donor's drops by need (it may go below zero and be refilled later);
 *   the move is realised by slicing the donor's own experts, biggest remaining count first
 *   (lowest id on ties), taking min(remaining, need) from each until need is covered; each
 *   slice (donor, receiver, expert, rows) is one entry of `moves`.
 * What no move took stays with the owner.  q[l*P + r] = entries of local expert l computed
 * by rank r.  [MF §3.1, App. A.2]: the plan keeps every selection and weight; rows are cut
 * into blocks of at most beta rows in the expert's stable order.  The ranks that compute
 * expert l take consecutive ranges of its segment in ascending rank order; the table lists
 * blocks rank by rank, then expert by expert: (rank, expert, first row, rows).
 * Pinned by: exact capacity and conservation invariants, move-count bound, hand-worked
 * golden plans (among them tied receivers and one donor serving two receivers, where the
 * second slice depends on the remaining counts), an exhaustive sweep of small count vectors
 * against brute-force properties, and move-for-move equality with a second, independent
 * statement of the greedy in Python (tests/plan_reference.py) on that sweep and on random
 * skewed counts. */
int oracle_plan(const int32_t* counts, int E, int begin, int stride, int E_loc, int P, int beta,
                int32_t* q, int32_t* moves, int32_t* n_moves, int max_moves,
                int32_t* blocks, int32_t* n_blocks, int max_blocks) {
    if (E_loc < 1 || P < 1 || E_loc % P != 0 || beta < 1 || stride < 1) return ORACLE_ERR_ARG;
    if (begin < 0 || begin + (int64_t)(E_loc - 1) * stride >= E) return ORACLE_ERR_ARG;
    const int G = E_loc / P;
    int64_t* n = (int64_t*)calloc((size_t)E_loc, sizeof(int64_t));
    int64_t* rem = (int64_t*)calloc((size_t)E_loc, sizeof(int64_t));
    int64_t* d = (int64_t*)calloc((size_t)P, sizeof(int64_t));
    int32_t* off = (int32_t*)calloc((size_t)E_loc + 1, sizeof(int32_t));
    int rc = ORACLE_OK;
    if (!n || !rem || !d || !off) { rc = ORACLE_ERR_DATA; goto done; }

    int64_t N = 0;
    for (int l = 0; l < E_loc; ++l) {
        n[l] = counts[begin + l * stride];
        rem[l] = n[l];
        N += n[l];
    }
    for (int r = 0; r < P; ++r) {
        int64_t cap = N / P + (r < N % P ? 1 : 0);
        int64_t load = 0;
        for (int l = r * G; l < (r + 1) * G; ++l) load += n[l];
        d[r] = load - cap;
    }
    for (int64_t i = 0; i < (int64_t)E_loc * P; ++i) q[i] = 0;

    int nm = 0;
    for (;;) {
        int recv = 0, donor = 0;
        for (int r = 1; r < P; ++r) {
            if (d[r] < d[recv]) recv = r;
            if (d[r] > d[donor]) donor = r;
        }
        if (d[recv] >= 0) break;
        int64_t need = -d[recv];
        d[donor] -= need;
        d[recv] = 0;
        while (need > 0) {
            int best = -1;
            for (int l = donor * G; l < (donor + 1) * G; ++l)
                if (rem[l] > 0 && (best < 0 || rem[l] > rem[best])) best = l;
            if (best < 0 || nm >= max_moves) { rc = ORACLE_ERR_DATA; goto done; }
            int64_t take = rem[best] < need ? rem[best] : need;
            q[(int64_t)best * P + recv] += (int32_t)take;
            rem[best] -= take;
            need -= take;
            moves[4 * nm + 0] = donor;
            moves[4 * nm + 1] = recv;
            moves[4 * nm + 2] = best;
            moves[4 * nm + 3] = (int32_t)take;
            ++nm;
        }
    }
    for (int l = 0; l < E_loc; ++l) q[(int64_t)l * P + l / G] += (int32_t)rem[l];
    *n_moves = nm;

    padded_offsets(counts, begin, stride, E_loc, beta, off);
    int nb = 0;
    for (int r = 0; r < P; ++r) {
        for (int l = 0; l < E_loc; ++l) {
            int64_t take = q[(int64_t)l * P + r];
            if (take <= 0) continue;
            int64_t first = off[l];
            for (int r2 = 0; r2 < r; ++r2) first += q[(int64_t)l * P + r2];
            for (int64_t j = 0; j * beta < take; ++j) {
                if (nb >= max_blocks) { rc = ORACLE_ERR_DATA; goto done; }
                int64_t rows = take - j * beta < beta ? take - j * beta : beta;
                blocks[4 * nb + 0] = r;
                blocks[4 * nb + 1] = l;
                blocks[4 * nb + 2] = (int32_t)(first + j * beta);
                blocks[4 * nb + 3] = (int32_t)rows;
                ++nb;
            }
        }
    }
    *n_blocks = nb;
done:
    free(n);
    free(rem);
    free(d);
    free(off);
    return rc;
}

/* ------------------------------------------------------- block-granular plan --- */

/* The block-granular planner of MegaFlux ([MF §3.1 "Problem formulation", "Bounded greedy
 * search"; App. A.1 "Candidate construction", "Refinement"]), over the same P logical ranks
 * and expert ownership as oracle_plan (rank r owns local experts r*G .. r*G + G - 1).
 *
 * Expert l's rows, in their stable order, are cut into b_l = ceil(n_l / beta) blocks of
 * beta rows (the last may be partial); load L_r counts blocks; tau = ceil(sum b_l / P).
 * Four searches start from the no-replica assignment q[l][owner(l)] = b_l.  A search runs
 * rounds; a round visits every rank that is over tau at its start once, in donor-priority
 * order (overload L_r - tau, or the rank's largest remaining home-expert block count;
 * larger first, lower rank on ties).  A visit scans the donor's home experts with blocks
 * left at home, most blocks first (lower id on ties), and ends when the donor is at tau or
 * the scan is done.  For each expert it moves single blocks while the donor is over tau and
 * the expert has blocks at home: to the least-loaded rank that already holds a copy of the
 * expert and is under tau, else to the least-loaded rank under tau with a free replica slot
 * (fewer than s copies of foreign experts), opening a new copy there -- in "one copy" mode
 * at most one new copy per expert per round, in "many copies" mode any number; ties go to
 * the lower rank.  The expert's fan-out stops when no receiver qualifies.  A search ends
 * after s + 2 rounds or a round that moved nothing.  Candidate order: (overload, one copy),
 * (overload, many), (home load, one copy), (home load, many).
 *
 * The candidate with the smallest maximum load wins, then the fewest replicas, then the
 * first in that order.  Refinement, at that maximum Lmax: replicas (copies of an expert on a
 * rank that does not own it), in increasing allocation at pass entry (then expert, then
 * rank), are removed when their whole allocation fits under Lmax on the owner or else on
 * the least-loaded other copy; then, at most sum b_l times, one block moves from the
 * most-loaded rank to the least-loaded rank (lowest rank on ties) while their loads differ
 * by more than one and both hold a copy of some expert with blocks on the former (the
 * owner always holds its experts; lowest such expert).
 *
 * Outputs as oracle_plan: q[l*P + r] = rows of expert l on rank r (the ranks holding l take
 * consecutive runs of its blocks in ascending rank order, so only the expert's last block is
 * partial); moves = one entry (owner, rank, expert, rows) per replica, expert then rank
 * ascending; blocks = (rank, expert, first row, rows), rank by rank, then expert by expert,
 * in block order.  Pinned by hand-worked plans (tests/golden/megaflux_plan_cases.json, one
 * of them with all four candidates tied on maximum load and replica count), closed forms (no
 * budget or a balanced start keep the no-replica assignment; an ample budget reaches tau),
 * invariants (conservation, budget, one partial block per expert, the refinement never
 * raising the maximum), and equality with a second, independent statement in Python
 * (tests/plan_reference.py) on random skewed counts. */
static void bp_search(const int64_t* b, int E_loc, int P, int G, int64_t tau, int s,
                      int by_overload, int many, int64_t* q, int64_t* L, int* repl,
                      unsigned char* opened, unsigned char* visited, int64_t* key, int* order) {
    for (int64_t i = 0; i < (int64_t)E_loc * P; ++i) q[i] = 0;
    for (int r = 0; r < P; ++r) { L[r] = 0; repl[r] = 0; }
    for (int l = 0; l < E_loc; ++l) {
        q[(int64_t)l * P + l / G] = b[l];
        L[l / G] += b[l];
    }
    for (int round = 0; round < s + 2; ++round) {
        int moved = 0;
        for (int l = 0; l < E_loc; ++l) opened[l] = 0;
        for (int r = 0; r < P; ++r) {
            visited[r] = 0;
            key[r] = -1;
            if (L[r] > tau) {
                if (by_overload) {
                    key[r] = L[r] - tau;
                } else {
                    key[r] = 0;
                    for (int l = r * G; l < (r + 1) * G; ++l)
                        if (q[(int64_t)l * P + r] > key[r]) key[r] = q[(int64_t)l * P + r];
                }
            }
        }
        for (;;) {
            int d = -1;
            for (int r = 0; r < P; ++r)
                if (!visited[r] && key[r] >= 0 && (d < 0 || key[r] > key[d])) d = r;
            if (d < 0) break;
            visited[d] = 1;
            if (L[d] <= tau) continue;
            /* the scan order is fixed at the start of the visit */
            int ns = 0;
            for (int l = d * G; l < (d + 1) * G; ++l)
                if (q[(int64_t)l * P + d] > 0) order[ns++] = l;
            for (int i = 1; i < ns; ++i) {  /* insertion sort: most blocks first, then lower id */
                int v = order[i], j = i;
                while (j > 0 && q[(int64_t)order[j - 1] * P + d] < q[(int64_t)v * P + d]) {
                    order[j] = order[j - 1];
                    --j;
                }
                order[j] = v;
            }
            for (int i = 0; i < ns && L[d] > tau; ++i) {
                const int l = order[i];
                int64_t* ql = q + (int64_t)l * P;
                while (ql[d] > 0 && L[d] > tau) {
                    int rcv = -1;
                    for (int r = 0; r < P; ++r)
                        if (r != d && ql[r] > 0 && L[r] < tau && (rcv < 0 || L[r] < L[rcv])) rcv = r;
                    if (rcv < 0 && (many || !opened[l])) {
                        for (int r = 0; r < P; ++r)
                            if (r != d && ql[r] == 0 && repl[r] < s && L[r] < tau &&
                                (rcv < 0 || L[r] < L[rcv]))
                                rcv = r;
                        if (rcv >= 0) {
                            repl[rcv] += 1;
                            opened[l] = 1;
                        }
                    }
                    if (rcv < 0) break;
                    ql[d] -= 1;
                    ql[rcv] += 1;
                    L[d] -= 1;
                    L[rcv] += 1;
                    moved = 1;
                }
            }
        }
        if (!moved) break;
    }
}

static int64_t bp_max(const int64_t* L, int P) {
    int64_t m = L[0];
    for (int r = 1; r < P; ++r) if (L[r] > m) m = L[r];
    return m;
}

static int64_t bp_replicas(const int64_t* q, int E_loc, int P, int G) {
    int64_t n = 0;
    for (int l = 0; l < E_loc; ++l)
        for (int r = 0; r < P; ++r)
            if (r != l / G && q[(int64_t)l * P + r] > 0) ++n;
    return n;
}

static int bp_key_cmp(const void* a, const void* b) {
    const int64_t* x = (const int64_t*)a;
    const int64_t* y = (const int64_t*)b;
    for (int i = 0; i < 3; ++i)
        if (x[i] != y[i]) return x[i] < y[i] ? -1 : 1;
    return 0;
}

int oracle_plan_blocks(const int32_t* counts, int E, int begin, int stride, int E_loc, int P,
                       int beta, int s, int32_t* q_out, int32_t* moves, int32_t* n_moves,
                       int max_moves, int32_t* blocks, int32_t* n_blocks, int max_blocks) {
    if (E_loc < 1 || P < 1 || E_loc % P != 0 || beta < 1 || stride < 1 || s < 0) return ORACLE_ERR_ARG;
    if (begin < 0 || begin + (int64_t)(E_loc - 1) * stride >= E) return ORACLE_ERR_ARG;
    const int G = E_loc / P;
    const int64_t EP = (int64_t)E_loc * P;
    int rc = ORACLE_OK;
    int64_t* n = (int64_t*)calloc((size_t)E_loc, sizeof(int64_t));
    int64_t* b = (int64_t*)calloc((size_t)E_loc, sizeof(int64_t));
    int64_t* q = (int64_t*)calloc((size_t)(4 * EP), sizeof(int64_t));
    int64_t* L = (int64_t*)calloc((size_t)(4 * P), sizeof(int64_t));
    int* repl = (int*)calloc((size_t)(4 * P), sizeof(int));
    unsigned char* opened = (unsigned char*)calloc((size_t)E_loc, 1);
    unsigned char* visited = (unsigned char*)calloc((size_t)P, 1);
    int64_t* key = (int64_t*)calloc((size_t)P, sizeof(int64_t));
    int* order = (int*)calloc((size_t)(G > 0 ? G : 1), sizeof(int));
    int64_t* rep = (int64_t*)calloc((size_t)(3 * EP), sizeof(int64_t));
    int32_t* off = (int32_t*)calloc((size_t)E_loc + 1, sizeof(int32_t));
    if (!n || !b || !q || !L || !repl || !opened || !visited || !key || !order || !rep || !off) {
        rc = ORACLE_ERR_DATA;
        goto done;
    }

    int64_t sum_b = 0;
    for (int l = 0; l < E_loc; ++l) {
        n[l] = counts[begin + l * stride];
        b[l] = (n[l] + beta - 1) / beta;
        sum_b += b[l];
    }
    const int64_t tau = (sum_b + P - 1) / P;

    /* the four searches */
    int best = 0;
    int64_t best_max = 0, best_rep = 0;
    for (int c = 0; c < 4; ++c) {
        bp_search(b, E_loc, P, G, tau, s, c < 2, c & 1, q + c * EP, L + c * P, repl + c * P,
                  opened, visited, key, order);
        const int64_t m = bp_max(L + c * P, P), nr = bp_replicas(q + c * EP, E_loc, P, G);
        if (c == 0 || m < best_max || (m == best_max && nr < best_rep)) {
            best = c;
            best_max = m;
            best_rep = nr;
        }
    }
    int64_t* qb = q + best * EP;
    int64_t* Lb = L + best * P;
    const int64_t Lmax = best_max;

    /* refinement 1: remove replicas whose allocation fits on the owner or another copy */
    int64_t nrep = 0;
    for (int l = 0; l < E_loc; ++l)
        for (int r = 0; r < P; ++r)
            if (r != l / G && qb[(int64_t)l * P + r] > 0) {
                rep[3 * nrep + 0] = qb[(int64_t)l * P + r];
                rep[3 * nrep + 1] = l;
                rep[3 * nrep + 2] = r;
                ++nrep;
            }
    qsort(rep, (size_t)nrep, 3 * sizeof(int64_t), bp_key_cmp);
    for (int64_t i = 0; i < nrep; ++i) {
        const int l = (int)rep[3 * i + 1], r = (int)rep[3 * i + 2], h = l / G;
        int64_t* ql = qb + (int64_t)l * P;
        const int64_t a = ql[r];
        if (a == 0) continue;
        int tgt = -1;
        if (Lb[h] + a <= Lmax) {
            tgt = h;
        } else {
            for (int r2 = 0; r2 < P; ++r2)
                if (r2 != r && r2 != h && ql[r2] > 0 && Lb[r2] + a <= Lmax &&
                    (tgt < 0 || Lb[r2] < Lb[tgt]))
                    tgt = r2;
        }
        if (tgt >= 0) {
            ql[tgt] += a;
            Lb[tgt] += a;
            ql[r] = 0;
            Lb[r] -= a;
        }
    }
    /* refinement 2: single blocks from the most- to the least-loaded rank */
    for (int64_t it = 0; it < sum_b; ++it) {
        int rmax = 0, rmin = 0;
        for (int r = 1; r < P; ++r) {
            if (Lb[r] > Lb[rmax]) rmax = r;
            if (Lb[r] < Lb[rmin]) rmin = r;
        }
        if (Lb[rmax] - Lb[rmin] <= 1) break;
        int lm = -1;
        for (int l = 0; l < E_loc && lm < 0; ++l)
            if (qb[(int64_t)l * P + rmax] > 0 && (rmin == l / G || qb[(int64_t)l * P + rmin] > 0)) lm = l;
        if (lm < 0) break;
        qb[(int64_t)lm * P + rmax] -= 1;
        qb[(int64_t)lm * P + rmin] += 1;
        Lb[rmax] -= 1;
        Lb[rmin] += 1;
    }

    /* rows per (expert, rank), replicas, and the block table */
    padded_offsets(counts, begin, stride, E_loc, beta, off);
    int nm = 0;
    for (int l = 0; l < E_loc; ++l) {
        int64_t pre = 0;
        for (int r = 0; r < P; ++r) {
            const int64_t k = qb[(int64_t)l * P + r];
            int64_t lo = pre * beta, hi = (pre + k) * beta;
            if (lo > n[l]) lo = n[l];
            if (hi > n[l]) hi = n[l];
            q_out[(int64_t)l * P + r] = (int32_t)(hi - lo);
            if (k > 0 && r != l / G) {
                if (nm >= max_moves) { rc = ORACLE_ERR_DATA; goto done; }
                moves[4 * nm + 0] = l / G;
                moves[4 * nm + 1] = r;
                moves[4 * nm + 2] = l;
                moves[4 * nm + 3] = (int32_t)(hi - lo);
                ++nm;
            }
            pre += k;
        }
    }
    *n_moves = nm;
    int nb = 0;
    for (int r = 0; r < P; ++r) {
        for (int l = 0; l < E_loc; ++l) {
            int64_t pre = 0;
            for (int r2 = 0; r2 < r; ++r2) pre += qb[(int64_t)l * P + r2];
            const int64_t k = qb[(int64_t)l * P + r];
            for (int64_t j = pre; j < pre + k; ++j) {
                if (nb >= max_blocks) { rc = ORACLE_ERR_DATA; goto done; }
                const int64_t rows = n[l] - j * beta < beta ? n[l] - j * beta : beta;
                blocks[4 * nb + 0] = r;
                blocks[4 * nb + 1] = l;
                blocks[4 * nb + 2] = (int32_t)(off[l] + j * beta);
                blocks[4 * nb + 3] = (int32_t)rows;
                ++nb;
            }
        }
    }
    *n_blocks = nb;
done:
    free(n); free(b); free(q); free(L); free(repl); free(opened); free(visited); free(key);
    free(order); free(rep); free(off);
    return rc;
}

/* -------------------------------------------------------------- MX formats --- */

/* Microscaled low-precision formats for the expert FFN ([MF §2.1 "Persistent MoE execution"]
 * and §4.1: MXFP4 weights, MXFP8 activations, FP32 accumulation, BF16 outputs; [MEP] cost
 * model: packed 4-bit elements plus one scale per 32 elements).  The element and scale
 * encodings are those of the OCP Microscaling Formats (MX) v1.0 specification:
 *   a block of 32 consecutive values shares one E8M0 scale 2^(code - 127) (code 255 = NaN is
 *   never produced), shared exponent = floor(log2(max |v|)) - emax_elem clamped to
 *   [-127, 127] (-127 for an all-zero block);
 *   elements: fmt 0 = FP8 E4M3 (bias 7, no infinities, max 448, emax 8), one byte each;
 *             fmt 1 = FP4 E2M1 (bias 1, values 0, 0.5, 1, 1.5, 2, 3, 4, 6, emax 2), two per byte,
 *             the lower-indexed element in the low nibble;
 *   element = v / scale rounded to the nearest representable value, ties to the even code,
 *   magnitudes beyond the largest value saturate to it.
 * Codes here come from the definition: the value of every non-negative code is computed and
 * the nearest is chosen. */
static double mx_elem_value(int fmt, int code) {
    const int s = fmt == 0 ? (code >> 7) & 1 : (code >> 3) & 1;
    const int e = fmt == 0 ? (code >> 3) & 15 : (code >> 1) & 3;
    const int m = fmt == 0 ? code & 7 : code & 1;
    const int mbits = fmt == 0 ? 3 : 1, bias = fmt == 0 ? 7 : 1;
    double v = e == 0 ? ldexp((double)m / (1 << mbits), 1 - bias)
                      : ldexp(1.0 + (double)m / (1 << mbits), e - bias);
    return s ? -v : v;
}

static int mx_max_code(int fmt) { return fmt == 0 ? 0x7E : 0x7; }  /* 448, 6 */

/* the values of the non-negative codes, filled once before any parallel use */
static double mx_table[2][128];
static int mx_table_ready = 0;
static void mx_fill_table(void) {
    if (mx_table_ready) return;
    for (int f = 0; f < 2; ++f)
        for (int c = 0; c <= mx_max_code(f); ++c) mx_table[f][c] = mx_elem_value(f, c);
    mx_table_ready = 1;
}
static int mx_emax(int fmt) { return fmt == 0 ? 8 : 2; }

/* nearest non-negative code to |v| (ties to the even code), then the sign */
static int mx_encode(int fmt, double v) {
    const double a = fabs(v);
    int best = 0;
    for (int c = 1; c <= mx_max_code(fmt); ++c) {
        const double dc = fabs(mx_table[fmt][c] - a), db = fabs(mx_table[fmt][best] - a);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    if (a > mx_table[fmt][mx_max_code(fmt)]) best = mx_max_code(fmt);
    const int sign = v < 0 && best != 0 ? 1 : 0;
    return best | (sign << (fmt == 0 ? 7 : 3));
}

/* src [rows, cols] (dt 0 = float32, 1 = bf16), cols a multiple of 32 ->
 * codes [rows, cols] (fmt 0) or [rows, cols / 2] (fmt 1), scales [rows, cols / 32]. */
int oracle_mx_quantize(const void* src, int dt, int64_t rows, int64_t cols, int fmt,
                       uint8_t* codes, uint8_t* scales) {
    if (rows < 0 || cols < 32 || cols % 32 != 0 || (dt != 0 && dt != 1) || (fmt != 0 && fmt != 1))
        return ORACLE_ERR_ARG;
    mx_fill_table();
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < cols / 32; ++b) {
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                const double v = fabs(load_elem(src, r * cols + b * 32 + j, dt));
                if (v > amax) amax = v;
            }
            int se = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);  /* amax = m * 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1 */
                se = ex - 1 - mx_emax(fmt);
                if (se < -127) se = -127;
                if (se > 127) se = 127;
            }
            scales[r * (cols / 32) + b] = (uint8_t)(se + 127);
            for (int j = 0; j < 32; ++j) {
                const int64_t i = r * cols + b * 32 + j;
                const int c = mx_encode(fmt, ldexp(load_elem(src, i, dt), -se));
                if (fmt == 0) {
                    codes[i] = (uint8_t)c;
                } else {
                    uint8_t* byte = codes + i / 2;
                    *byte = (uint8_t)((i & 1) ? ((*byte & 0x0F) | (c << 4)) : ((*byte & 0xF0) | c));
                }
            }
        }
    }
    return ORACLE_OK;
}

static double mx_value(const uint8_t* codes, const uint8_t* scales, int64_t cols, int fmt, int64_t r,
                       int64_t c) {
    const int64_t i = r * cols + c;
    const int code = fmt == 0 ? codes[i] : ((codes[i / 2] >> ((i & 1) * 4)) & 0xF);
    const int mag = code & (fmt == 0 ? 0x7F : 0x7), neg = code != mag;
    const double v = ldexp(mx_table[fmt][mag], (int)scales[r * (cols / 32) + c / 32] - 127);
    return neg ? -v : v;
}

int oracle_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                         int fmt, double* out) {
    if (rows < 0 || cols < 32 || cols % 32 != 0 || (fmt != 0 && fmt != 1)) return ORACLE_ERR_ARG;
    mx_fill_table();
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = mx_value(codes, scales, cols, fmt, r, c);
    return ORACLE_OK;
}

/* SwiGLU expert FFN in the MX formats ([MF §4.1 Platform and configurations]: MXFP4 weights,
 * MXFP8 activations, FP32 accumulation, BF16 outputs), for a list of rows.  xq/xs: the layer
 * input rows in MXFP8 (E4M3 codes [*, H], scales [*, H/32]); w1q/w1s: W1 in MXFP4 ([E_loc, 2I,
 * H/2] packed, scales [E_loc, 2I, H/32]; rows 0..I-1 gate, I..2I-1 up); w2q/w2s: W2 in MXFP4
 * ([E_loc, H, I/2], [E_loc, H, I/32]).  Row j of the list is row rows[j] of xq, expert
 * row_expert[j]:
 *   g_i, u_i = dot products of the dequantized values in double;
 *   a_i = g_i / (1 + exp(-g_i)) * u_i, quantized to MXFP8 per 32 columns -> actq [n, I], acts;
 *   yp[j][h] = bf16(sum_i deq(actq)[i] * deq(W2[l][h][i]))  (double). */
int oracle_ffn_mx_rows(const uint8_t* xq, const uint8_t* xs, int H, int I, const uint8_t* w1q,
                       const uint8_t* w1s, const uint8_t* w2q, const uint8_t* w2s,
                       const int32_t* rows, const int32_t* row_expert, int n, uint8_t* actq,
                       uint8_t* acts, uint16_t* yp) {
    if (H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0 || n < 0) return ORACLE_ERR_ARG;
    mx_fill_table();
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int j = 0; j < n; ++j) {
        const int64_t p = rows[j], l = row_expert[j];
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        if (!a) { bad = 1; continue; }
        const uint8_t* w1qe = w1q + l * 2 * I * (int64_t)(H / 2);
        const uint8_t* w1se = w1s + l * 2 * I * (int64_t)(H / 32);
        for (int i = 0; i < I; ++i) {
            double g = 0.0, u = 0.0;
            for (int h = 0; h < H; ++h) {
                const double xv = mx_value(xq, xs, H, 0, p, h);
                g += xv * mx_value(w1qe, w1se, H, 1, i, h);
                u += xv * mx_value(w1qe, w1se, H, 1, I + i, h);
            }
            a[i] = g / (1.0 + exp(-g)) * u;
        }
        /* the activation row in MXFP8: the same rule as oracle_mx_quantize, from double */
        for (int b = 0; b < I / 32; ++b) {
            double amax = 0.0;
            for (int k = 0; k < 32; ++k) if (fabs(a[b * 32 + k]) > amax) amax = fabs(a[b * 32 + k]);
            int se = -127;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);
                se = ex - 1 - mx_emax(0);
                if (se < -127) se = -127;
                if (se > 127) se = 127;
            }
            acts[(int64_t)j * (I / 32) + b] = (uint8_t)(se + 127);
            for (int k = 0; k < 32; ++k)
                actq[(int64_t)j * I + b * 32 + k] = (uint8_t)mx_encode(0, ldexp(a[b * 32 + k], -se));
        }
        const uint8_t* w2qe = w2q + l * (int64_t)H * (I / 2);
        const uint8_t* w2se = w2s + l * (int64_t)H * (I / 32);
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int i = 0; i < I; ++i)
                acc += mx_value(actq, acts, I, 0, j, i) * mx_value(w2qe, w2se, I, 1, h, i);
            yp[(int64_t)j * H + h] = oracle_double_to_bf16(acc);
        }
        free(a);
    }
    return bad ? ORACLE_ERR_DATA : ORACLE_OK;
}

/* ------------------------------------------------------------------- expert FFN --- */

/* SwiGLU expert FFN for a list of rows.  [MF §2.1, §4.1]: FC1 produces gate and up
 * projections, the activation is SiLU(gate) * up, FC2 projects back to H; accumulation is
 * in high precision and outputs are BF16.
 *
 * Row j of the list is row rows[j] of xp ([*, H]); it uses local expert row_expert[j]:
 *   W1 is [E_loc, 2I, H] (rows 0..I-1 gate, I..2I-1 up), W2 is [E_loc, H, I].
 *   g_i = sum_h xp[p][h] * W1[l][i][h],  u_i = sum_h xp[p][h] * W1[l][I+i][h]   (double)
 *   act[j][i] = round(g_i / (1 + exp(-g_i)) * u_i)
 *   yp[j][h]  = round(sum_i act[j][i] * W2[l][h][i])                            (double)
 * round = bf16 nearest-even when dt == 1, float32 when dt == 0.  act is [n, I], yp [n, H].
 * Pinned by: E=1, K=1 against a dense SwiGLU written with torch.matmul in float64. */
int oracle_ffn_rows(const void* xp, int dt, int H, int I, const void* w1, const void* w2,
                    const int32_t* rows, const int32_t* row_expert, int n, void* act, void* yp) {
    if (H < 1 || I < 1 || n < 0 || (dt != 0 && dt != 1)) return ORACLE_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int j = 0; j < n; ++j) {
        int64_t p = rows[j];
        int64_t l = row_expert[j];
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        if (!a) { bad = 1; continue; }
        const int64_t w1_base = l * 2 * (int64_t)I * H;
        for (int i = 0; i < I; ++i) {
            double g = 0.0, u = 0.0;
            for (int h = 0; h < H; ++h) {
                double xv = load_elem(xp, p * H + h, dt);
                g += xv * load_elem(w1, w1_base + (int64_t)i * H + h, dt);
                u += xv * load_elem(w1, w1_base + (int64_t)(I + i) * H + h, dt);
            }
            double v = g / (1.0 + exp(-g)) * u;
            store_elem(act, (int64_t)j * I + i, dt, v);
            a[i] = load_elem(act, (int64_t)j * I + i, dt); /* FC2 consumes the stored value */
        }
        const int64_t w2_base = l * (int64_t)H * I;
        for (int h = 0; h < H; ++h) {
            double y = 0.0;
            for (int i = 0; i < I; ++i) y += a[i] * load_elem(w2, w2_base + (int64_t)h * I + i, dt);
            store_elem(yp, (int64_t)j * H + h, dt, y);
        }
        free(a);
    }
    return bad ? ORACLE_ERR_DATA : ORACLE_OK;
}

/* The FFN over a block table: every row of every block (rank, expert, first, rows) is
 * computed with that block's expert, results written at the same row of act [*, I] and
 * yp [*, H] (full-size arrays indexed by permuted row). */
int oracle_ffn_blocks(const void* xp, int dt, int H, int I, const void* w1, const void* w2,
                      const int32_t* blocks, int n_blocks, void* act, void* yp) {
    int64_t total = 0;
    for (int b = 0; b < n_blocks; ++b) total += blocks[4 * b + 3];
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
    int32_t* ex = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
    size_t es = dt == 1 ? 2 : 4;
    void* a = malloc(es * (size_t)(total > 0 ? total : 1) * (size_t)I);
    void* y = malloc(es * (size_t)(total > 0 ? total : 1) * (size_t)H);
    int rc = ORACLE_OK;
    if (!rows || !ex || !a || !y) { rc = ORACLE_ERR_DATA; goto done; }
    int64_t j = 0;
    for (int b = 0; b < n_blocks; ++b)
        for (int m = 0; m < blocks[4 * b + 3]; ++m) {
            rows[j] = blocks[4 * b + 2] + m;
            ex[j] = blocks[4 * b + 1];
            ++j;
        }
    rc = oracle_ffn_rows(xp, dt, H, I, w1, w2, rows, ex, (int)total, a, y);
    if (rc != ORACLE_OK) goto done;
    for (int64_t k = 0; k < total; ++k) {
        memcpy((char*)act + (int64_t)rows[k] * I * es, (char*)a + k * I * es, (size_t)I * es);
        memcpy((char*)yp + (int64_t)rows[k] * H * es, (char*)y + k * H * es, (size_t)H * es);
    }
done:
    free(rows);
    free(ex);
    free(a);
    free(y);
    return rc;
}

/* ---------------------------------------------------------------------- combine --- */

/* Routing-weight combine.  [MF §1]: expert outputs are mixed with the routing weights;
 * [MF §2.1]: the top-k sum is a separate step; [MF App. A.2]: token ids, top-k positions
 * and weights are kept for it.
 *   out[t][h] = round( sum over k = 0..K-1 with entry_pos[t*K+k] >= 0 of
 *                      w[t][k] * yp[entry_pos[t*K+k]][h] )      (double, k ascending)
 * A token with no local entry gets 0.  round as in oracle_ffn_rows.
 * Pinned by: K = 1 reproduces the expert row; no local entry gives 0; equal-logit K = E
 * gives the mean of all experts' outputs. */
int oracle_combine(const void* yp, int dt, const float* w, const int32_t* entry_pos, int T, int H,
                   int K, void* out) {
    if (T < 1 || H < 1 || K < 1 || (dt != 0 && dt != 1)) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            double s = 0.0;
            for (int k = 0; k < K; ++k) {
                int64_t p = entry_pos[(int64_t)t * K + k];
                if (p < 0) continue;
                s += (double)w[(int64_t)t * K + k] * load_elem(yp, p * H + h, dt);
            }
            store_elem(out, (int64_t)t * H + h, dt, s);
        }
    }
    return ORACLE_OK;
}
