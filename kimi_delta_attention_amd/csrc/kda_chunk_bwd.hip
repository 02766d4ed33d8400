// kda_chunk_bwd.hip -- chunked KDA backward (not built yet in this revision).
#include "kda_chunk_common.hpp"

namespace kda {

size_t chunk_bwd_workspace(const ChunkParams&) { return 0; }

hipError_t launch_chunk_bwd(const ChunkParams&, const ChunkGrads&, void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace kda
