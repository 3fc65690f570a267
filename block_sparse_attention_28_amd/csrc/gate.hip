// gate.hip -- gate scores of one decode step (standalone launch).
//
// The body, and the description of the operation and of its gfx950 mapping,
// are in gate_items.hpp; the fused decode step runs the same body.
#include "gate_items.hpp"
#include "seer_host.hpp"

namespace seer {

// One 1024-thread workgroup per part of a pair: the pair's complete blocks
// are dealt evenly over `parts` workgroups (the last one also writes -inf past
// them).  u is formed in GateU's one fixed order, as in every other gate body
// (here threads 256..511 hold the Wk rows), so the scores match the fused
// step's bit for bit.
template <int D, int QB>
__global__ __launch_bounds__(1024) void gate_scores_kernel(const GateArgs ga, int parts) {
    __shared__ GateSmem<D> sm;
    const int pair = blockIdx.x / parts, part = blockIdx.x % parts;
    int L = ga.seqlens[pair / ga.Hkv];
    L = L < 0 ? 0 : L;
    int nc = L / ga.block_size;
    nc = nc > ga.nb_max ? ga.nb_max : nc;
    const int jb = (int)((int64_t)part * nc / parts);
    const int je = part == parts - 1 ? ga.nb_max : (int)((int64_t)(part + 1) * nc / parts);
    gate_rows_item<D, LaunchMem, QB, 1024>(ga, pair, jb, je, sm);
}

// Query rows in flight: the group size rounded up to 1, 2, 4 or 8.
template <int D>
static void launch_gate(const GateArgs &ga, int pairs, int parts, hipStream_t stream) {
    const dim3 grid((unsigned)(pairs * parts));
    if (ga.G == 1)
        gate_scores_kernel<D, 1><<<grid, 1024, 0, stream>>>(ga, parts);
    else if (ga.G == 2)
        gate_scores_kernel<D, 2><<<grid, 1024, 0, stream>>>(ga, parts);
    else if (ga.G <= 4)
        gate_scores_kernel<D, 4><<<grid, 1024, 0, stream>>>(ga, parts);
    else
        gate_scores_kernel<D, 8><<<grid, 1024, 0, stream>>>(ga, parts);
}

}  // namespace seer

using namespace seer;

extern "C" int seer_gate_scores(const seer_bf16 *q, int64_t sq_b, int64_t sq_h, const seer_bf16 *wq,
                                const seer_bf16 *wk, int dg, const float *kpool, int nb_max, const int32_t *seqlens,
                                int B, int Hq, int Hkv, int d, int block_size, float gate_scale, float *scores,
                                hipStream_t stream) {
    if (!q || !wq || !wk || !seqlens || !scores) return SEER_ERR_INVALID_ARG;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || nb_max < 0 || block_size <= 0 || dg < 1 || dg > 256 ||
        !rows_aligned16(q, sq_h) || !rows_aligned16(q, sq_b) || !aligned16(wq) || !aligned16(wk) ||
        !(gate_scale == gate_scale))
        return SEER_ERR_INVALID_ARG;
    if (nb_max > 0 && (!kpool || !aligned16(kpool))) return SEER_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return SEER_ERR_UNSUPPORTED;
    if ((int64_t)B * Hkv > 65535) return SEER_ERR_INVALID_ARG;
    if (nb_max == 0) return SEER_OK;
    GateArgs ga{q, sq_b, sq_h, wq, wk, dg, Hq / Hkv, Hkv, gate_scale, kpool, nb_max, seqlens, block_size, scores};
    // Enough parts per pair for about one workgroup per compute unit, each with
    // at least 128 rows.
    const int pairs = B * Hkv;
    int parts = device_cu_count() / pairs;
    const int max_parts = nb_max / 128;
    parts = parts > max_parts ? max_parts : parts;
    parts = parts < 1 ? 1 : (parts > 64 ? 64 : parts);
    if (d == 128)
        launch_gate<128>(ga, pairs, parts, stream);
    else
        launch_gate<64>(ga, pairs, parts, stream);
    return launch_status();
}
