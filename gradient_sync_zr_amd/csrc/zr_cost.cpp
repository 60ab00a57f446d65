// alpha-beta cost model of ring, tree and naive all-reduce and of the
// segmented (pipelined) ring broadcast (CMU 11-868 lecture 14 notes, 3.1
// pipelined broadcast and 3.4 the alpha-beta model; 4.4 the data-parallel
// speedup). Host arithmetic only, no GPU. A message of n bytes costs
// alpha + n / beta; every formula below charges one message per round.
#include <cmath>
#include <limits>

#include "zr.h"

namespace {

constexpr double kNaN = std::numeric_limits<double>::quiet_NaN();

bool bad(int K, double bytes, double alpha, double beta) {
    return K < 1 || !(bytes >= 0) || !(alpha >= 0) || !(beta > 0);
}

int ceil_log2(int K) {
    int L = 0;
    while ((1 << L) < K) ++L;
    return L;
}

}  // namespace

extern "C" {

// Ring all-reduce: 2(K-1) rounds, each moving one chunk of bytes / K.
double zr_cost_ring_allreduce(int K, double bytes, double alpha, double beta) {
    if (bad(K, bytes, alpha, beta)) return kNaN;
    return 2.0 * (K - 1) * (alpha + bytes / (K * beta));
}

// Ring reduce-scatter (or all-gather) alone: K-1 rounds of one chunk.
double zr_cost_ring_reduce_scatter(int K, double bytes, double alpha, double beta) {
    if (bad(K, bytes, alpha, beta)) return kNaN;
    return (K - 1) * (alpha + bytes / (K * beta));
}

// Binary tree: reduce up and broadcast down, ceil(log2 K) rounds each, whole
// message per round.
double zr_cost_tree_allreduce(int K, double bytes, double alpha, double beta) {
    if (bad(K, bytes, alpha, beta)) return kNaN;
    return 2.0 * ceil_log2(K) * (alpha + bytes / beta);
}

// Everyone sends to one device, which sends the sum back: two rounds whose
// transfer time is that device's K-1 messages.
double zr_cost_naive_allreduce(int K, double bytes, double alpha, double beta) {
    if (bad(K, bytes, alpha, beta)) return kNaN;
    return 2.0 * (alpha + (K - 1) * bytes / beta);
}

// Ring broadcast of `bytes` cut into S segments: the first segment needs
// K-1 hops, the others follow one step behind, K-2+S steps of bytes/S each.
// S = 1 is the unsegmented broadcast, (K-1)(alpha + bytes/beta).
double zr_cost_pipelined_broadcast(int K, double bytes, int segments, double alpha, double beta) {
    if (bad(K, bytes, alpha, beta) || K < 2 || segments < 1) return kNaN;
    return (K - 2 + segments) * (alpha + bytes / (segments * beta));
}

// The power-of-two segment count in [1, max_segments] with the smallest
// pipelined-broadcast time (the earliest on ties); its time in *time.
int zr_cost_best_broadcast_segments(int K, double bytes, double alpha, double beta,
                                    int max_segments, double* time) {
    if (bad(K, bytes, alpha, beta) || K < 2 || max_segments < 1) return -1;
    int best = 1;
    double t_best = zr_cost_pipelined_broadcast(K, bytes, 1, alpha, beta);
    for (long s = 2; s <= max_segments; s *= 2) {
        const double t = zr_cost_pipelined_broadcast(K, bytes, (int)s, alpha, beta);
        if (t < t_best) {
            t_best = t;
            best = (int)s;
        }
    }
    if (time) *time = t_best;
    return best;
}

// Message size at which ring and tree all-reduce take equal time (bytes):
// 2(K-1)(a + n/(K b)) = 2L(a + n/b), L = ceil(log2 K).
double zr_cost_ring_tree_crossover(int K, double alpha, double beta) {
    if (bad(K, 0.0, alpha, beta)) return kNaN;
    const double L = ceil_log2(K);
    const double den = L - (K - 1.0) / K;
    if (den <= 0) return kNaN;
    return (K - 1.0 - L) * alpha * beta / den;
}

// Message size at which ring and naive all-reduce take equal time (bytes):
// 2(K-1)(a + n/(K b)) = 2(a + (K-1) n / b).
double zr_cost_ring_naive_crossover(int K, double alpha, double beta) {
    if (bad(K, 0.0, alpha, beta) || K < 2) return kNaN;
    return (K - 2.0) * K * alpha * beta / ((K - 1.0) * (K - 1.0));
}

// Data-parallel speedup without overlap: t1 / (t1 / K + ring all-reduce of
// the gradient bytes).
double zr_cost_dp_speedup(int K, double t1, double grad_bytes, double alpha, double beta) {
    if (bad(K, grad_bytes, alpha, beta) || !(t1 > 0)) return kNaN;
    return t1 / (t1 / K + zr_cost_ring_allreduce(K, grad_bytes, alpha, beta));
}

}  // extern "C"
