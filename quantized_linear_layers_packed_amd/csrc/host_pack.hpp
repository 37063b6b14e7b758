// Pieces of the host encoders shared between the round-to-nearest encoders
// and the second-order (Hessian-aware) encoders.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

namespace qlin {

// Mask of the n entries first in the order (-key, index).
template <typename T>
std::vector<uint8_t> top_n_mask(const T* key, size_t total, int64_t n);

// Round-to-nearest statistics of one group of G fp32 weights in the 4-bit
// storage: lo = min(0, min w), hi = max(0, max w), S = fp16((hi - lo) / 15)
// (1 if that is 0), z = clamp(rint(-lo / S), 0, 15); s = float(S).
void w4_group_stats(const float* w, int G, uint16_t* S, float* s, float* z);
// Code of one weight against those statistics: clamp(rint(w / s) + z, 0, 15).
uint32_t w4_code(float w, float s, float z);

// SpQR storage of W with the outlier positions given by `mask` (N*K bytes,
// nonzero = outlier): CSR of the outliers, bi-level 3-bit encode of the rest.
void spqr_encode_masked(const float* W, int N, int K, const uint8_t* mask,
                        uint32_t* codes, uint32_t* stats1, uint16_t* stats2,
                        int32_t* row_ptr, int32_t* col_idx, uint16_t* vals, int64_t* nnz_out);

}  // namespace qlin
