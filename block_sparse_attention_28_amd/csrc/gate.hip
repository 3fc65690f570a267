// gate.hip -- gate scores of one decode step (standalone launch).
//
// The body, and the description of the operation and of its gfx950 mapping,
// are in gate_items.hpp; the fused decode step runs the same body.
#include "gate_items.hpp"
#include "seer_host.hpp"

namespace seer {

template <int D, int QB>
__global__ __launch_bounds__(256) void gate_scores_kernel(const GateArgs ga) {
    __shared__ GateSmem<D> sm;
    gate_chunk_item<D, LaunchMem, QB>(ga, blockIdx.x, blockIdx.y, sm);
}

// Query rows in flight: the group size rounded up to 1, 2, 4 or 8.
template <int D>
static void launch_gate(const GateArgs &ga, dim3 grid, hipStream_t stream) {
    if (ga.G == 1)
        gate_scores_kernel<D, 1><<<grid, 256, 0, stream>>>(ga);
    else if (ga.G == 2)
        gate_scores_kernel<D, 2><<<grid, 256, 0, stream>>>(ga);
    else if (ga.G <= 4)
        gate_scores_kernel<D, 4><<<grid, 256, 0, stream>>>(ga);
    else
        gate_scores_kernel<D, 8><<<grid, 256, 0, stream>>>(ga);
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
    if (d == 128)
        launch_gate<128>(ga, dim3((nb_max + GateCfg<128>::RPB - 1) / GateCfg<128>::RPB, B * Hkv), stream);
    else
        launch_gate<64>(ga, dim3((nb_max + GateCfg<64>::RPB - 1) / GateCfg<64>::RPB, B * Hkv), stream);
    return launch_status();
}
