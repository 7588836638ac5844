// Internal interface of the compressors.
#pragma once
#include "common.h"

namespace vc {

vc_status compress_layout(const vc_compress_desc* d, vc_compress_layout* L);
vc_status compress_ws_bytes(const vc_compress_desc* d, size_t* ws);
vc_status compress_run(const vc_compress_desc* d, const void* k, const void* v, const void* q_obs, void* out,
                       size_t out_bytes, void* ws, size_t ws_bytes, hipStream_t s);
// Token drop: copy the rows of src [L*Hkv][src_cap] that were not kept (positions below
// seq_len), compacted in position order, for (layer*head) rows [lh0, lh0 + n_lh) into
// dst [n_lh][dst_cap].
vc_status gather_dropped(const vc_compress_desc* d, const void* comp, const void* src, int src_cap, int lh0, int n_lh,
                         void* dst, int dst_cap, hipStream_t s);

}  // namespace vc
