// Internal interface of the compressors.
#pragma once
#include "common.h"

namespace vc {

vc_status compress_layout(const vc_compress_desc* d, vc_compress_layout* L);
vc_status compress_ws_bytes(const vc_compress_desc* d, size_t* ws);
vc_status compress_run(const vc_compress_desc* d, const void* k, const void* v, const void* q_obs, void* out,
                       size_t out_bytes, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace vc
