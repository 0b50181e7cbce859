// Status codes and the thread-local last-error text shared by the host files.
#pragma once

namespace mesh_attn {

// Records msg as this thread's last error and returns status.
int fail(int status, const char* msg);
void clear_error();

}  // namespace mesh_attn
