#include "fa_common.h"
#include "fa_launch.h"
namespace fa {
hipError_t launch_backward(const BwdArgs&) { return hipErrorNotSupported; }
long long backward_grid_size(int B, int H, int N) { return (long long)B * H * ((N + 127) / 128); }
}
