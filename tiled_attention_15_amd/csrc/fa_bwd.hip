// fa_bwd.hip -- attention backward for gfx950 (MI355X).
//
// Gradients of the loss sum(O * dO) with respect to Q, K and V.  The score
// and probability tiles are recomputed from Q, K and the forward's row
// log-sum-exp instead of being stored ("ops-transformer FlashAttention
// operator in practice" (ai6s.net), section 2, table of core optimisations:
// recomputation in the backward pass; "FlashAttention-2 on Ascend NPU"
// (2048ai.net), section 6.2: the forward keeps no attention matrix, so the
// backward recomputes it).  dQ is computed deterministically, the
// "deterministic" mode of "catlass FlashAttention tuning for a 13B service"
// (gsyq.cn), backward-pass section: a second kernel owns each dQ row and sums
// its key tiles in a fixed order (scores recomputed once more), so results
// are bitwise reproducible.  The page's faster non-deterministic mode (dQ
// accumulated with float atomics while dK/dV are computed) is not provided:
// on MI355X it measured 1.8x slower, and with its atomics removed it only
// tied this mode (the dQ product, its LDS round trip and barrier inside the
// dK/dV kernel cost what the separate pass costs).
//
// Per (batch, head), with P_ij = exp(scale q_i.k_j - lse_i) (0 where hidden)
// and D_i = dO_i . O_i (= sum_j P_ij dP_ij):
//   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i),
//   dQ_i = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i.
//
// Kernels:
//   bwd_pre      D_i for every row;
//   bwd_dkdv_pp  (D = 128, no mask or dropout) one workgroup of 8 waves per
//                256-key block: two groups of four waves (128 keys each, 32
//                per wave) alternate between a matrix phase (dV^T += dO^T P,
//                dK^T += Q^T dS of the previous 32-query tile, then S = Q K^T
//                and dP = dO V^T of this one) and an elementwise phase (P and
//                dS), as the forward's two groups do; Q/dO tiles and their
//                lse and D_i stream through a three-stage LDS ring shared by
//                both groups;
//   bwd_dkdv     (D = 64, D = 256, and with a mask or dropout) one workgroup of
//                4 waves per 128-key block with the same products per tile and
//                a double-buffered Q/dO ring;
//   bwd_dq       one workgroup per 128-query block (32 queries per wave, Q and
//                dO resident); 64-key tiles of K and V stream through LDS;
//                S^T = K Q^T, dP^T = V dO^T, then dQ^T += K^T dS^T.
// In the dK/dV kernels the key block sits in LDS and V of a wave's 32 keys in
// registers; queries are on MFMA rows and keys on columns for S and dP; P and
// dS go from the accumulators, packed to 16 bits, straight into the B
// operands of dV^T and dK^T, whose A operands dO^T and Q^T come from LDS by
// transposing reads (ds_read_b64_tr_b16).  All tiles are loaded straight into
// LDS (buffer_load ... lds).
//
// The operand layouts and LDS helpers are in fa_tile.h.
#include "fa_bwd_kernels.h"

namespace fa {
namespace bwd {

hipError_t launch_bwd(const BwdParams& p, int D, int dtype, int causal,
                      hipStream_t stream) {
    if (D == 256) return launch_bwd256(p, dtype, causal, stream);
    if (D == 64) {
        if (dtype == 0) return causal ? run<64, 0, true>(p, stream) : run<64, 0, false>(p, stream);
        return causal ? run<64, 1, true>(p, stream) : run<64, 1, false>(p, stream);
    }
    if (dtype == 0) return causal ? run<128, 0, true>(p, stream) : run<128, 0, false>(p, stream);
    return causal ? run<128, 1, true>(p, stream) : run<128, 1, false>(p, stream);
}

}  // namespace bwd
}  // namespace fa
